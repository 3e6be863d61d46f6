"""MI355X-native hot path of one GPU's share of a Mixture-of-Experts layer forward."""
