"""CPU oracle of the Step-5 sparse-indexer path (test infrastructure only)."""
