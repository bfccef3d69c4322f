"""CPU oracle of the MoE layer -- test infrastructure only (tests, smoke check,
benchmark CPU baseline).  The GPU path never imports this package."""
