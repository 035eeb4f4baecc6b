// The decode kernels' launchers and instantiations, compiled as a unit of
// their own (the kernel templates are those of kernels_expert.hip): the two
// halves of the expert kernels build in parallel.
#define STRATA_DECODE_UNIT
#include "kernels_expert.hip"
