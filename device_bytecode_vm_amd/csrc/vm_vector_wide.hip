// The wide build of the VECTOR VM: one tile register of NV_WIDE chunks per
// lane instead of three of NV_MAX, so a tile holds twice the columns per lane
// (rows up to T_LANES * NV_WIDE * VEC elements, two rows per tile where the
// standard build fits one).  Same interpreter, same handlers; kernels and
// launch functions carry a _wide suffix.
#define DVM_WIDE 1
#include "vm_vector.hip"
