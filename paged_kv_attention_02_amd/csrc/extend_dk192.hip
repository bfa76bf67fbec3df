// forward_extend at 192-wide keys and 128-wide values over a bf16 cache: the
// MFMA kernel's instantiations for these widths (launch_extend_dk192), compiled in a
// translation unit of their own with the compiler's max-ILP scheduling
// strategy (see paged_kv_attention_02_amd/build.py).  The kernel itself is
// the one in extend.hip.
#define PKA_EXTEND_DK192_TU
#include "extend.hip"
