"""MI355X-native Longformer window + global attention forward (``lwattn``)."""
