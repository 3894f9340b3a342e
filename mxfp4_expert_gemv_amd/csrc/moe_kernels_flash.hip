// moe_kernels_flash.hip -- the layer kernels and their launcher compiled ahead of time for one layer
// shape: hidden 2560, 512 routed experts, top-8, one shared expert, expert width 768 (the MoE layer
// of the pages' model: tanhow.com, "NVIDIA 在单台 DGX Spark 上叠加三项优化...", section "Ling 3.0 是什么").
// The shape is folded in at compile time, as in the run-time compiled kernels (MOE_F_JIT), so that the
// compiler resolves the divisions, loop bounds and tile counts that the shape-generic build takes
// from the kernel arguments.  The input normalisation (MOE_SHAPE_NORM, left undefined) stays a
// run-time argument.  Everything lands in namespace moe::flash; handles of this shape use it unless
// created with MOE_F_GENERIC.
#define MOE_SHAPE_H 2560
#define MOE_SHAPE_E 512
#define MOE_SHAPE_K 8
#define MOE_SHAPE_S 1
#define MOE_SHAPE_I 768
// the gate/up and down geometry that shape implies (Shape::bpl, ksub, iters): the only instances built
#define MOE_FIXED_BPL 8
#define MOE_FIXED_KSUB 8
#define MOE_FIXED_ITERS 3
#define MOE_KERNELS_NS_BEGIN \
    namespace moe {          \
    namespace flash {
#define MOE_KERNELS_NS_END \
    }                      \
    }
#include "moe_kernels.hip"

namespace moe {
namespace flash {
bool shape_matches(const Shape& sh) {
    return sh.H == MOE_SHAPE_H && sh.E == MOE_SHAPE_E && sh.k == MOE_SHAPE_K && sh.S == MOE_SHAPE_S &&
           sh.I == MOE_SHAPE_I && sh.bpl() == MOE_FIXED_BPL && sh.ksub() == MOE_FIXED_KSUB &&
           sh.iters() == MOE_FIXED_ITERS;
}
}  // namespace flash
}  // namespace moe
