"""Development tools behind the planner's cost model: the timing sweep
(GPU) and the fit of the model to its results (CPU).  Nothing in the library
imports them."""
