"""MI355X-native MoE expert-parallel dispatch layout, dispatch pack and combine."""
