// bounds.hpp - the bounds-check build's hooks (FNO_BOUNDS_CHECK defined).
//
// Every launcher states, before it launches, the index ranges its kernel
// will touch: each buffer's span derived from the argument block exactly as
// the kernel indexes it, and the kernel's structural assumptions (tile
// counts, grid no larger than the work, LDS within the chip's 160 KiB and no
// smaller than the kernel's layout). In the bounds-check build the host code
// runs on the CPU against a recording runtime whose allocations are known,
// and a span outside every live allocation, or a broken assumption, is
// reported (the TurboFNO write-up's debugging section, 6.1, describes the
// failure class this guards against: an out-of-range twiddle index). In the
// library build the hooks compile to nothing.

#pragma once

#ifdef FNO_BOUNDS_CHECK

#include <cstddef>

namespace fno {

struct PlaneFwdArgs;
struct PlaneInvArgs;
struct PlaneMxFwdArgs;
struct PlaneMxInvArgs;
struct AxisArgs;
struct ContractArgs;
struct GradWArgs;
struct WeightsArgs;
struct FusedShape;

namespace bounds {
// [p, p + n) inside one live allocation of the recording runtime (n = 0: true)
bool inside(const void *p, size_t n);
// a broken span or assumption of launch `launch`
void report(const char *launch, const char *what);
}  // namespace bounds

void check_plane_fwd(const PlaneFwdArgs &a, int MP, int rpt, int dtype, size_t lds);
void check_plane_inv(const PlaneInvArgs &a, int MP, int rpt, int dtype, size_t lds);
void check_plane_mx_fwd(const PlaneMxFwdArgs &a, int grid, int dtype, size_t lds, bool two);
void check_plane_mx_inv(const PlaneMxInvArgs &a, int grid, int dtype, size_t lds, bool cols);
void check_axis(const AxisArgs &a, bool fwd);
void check_contract(const ContractArgs &a, int dtype, bool mx);
void check_contract_adj(const ContractArgs &a, int bb, int S, size_t wave_bytes, size_t stage_bytes);
void check_grad_w(const GradWArgs &a, int dtype);
void check_conj_transpose(const void *w, const void *wh, int K, int Ci, int Co, int dtype);
void check_weights_repack(const WeightsArgs &a, int dtype);
void check_layer_fused(const FusedShape &f, const void *args, int grid, size_t lds);
void check_channel_mix(const void *x, const void *A, const void *bias, const void *add, const void *y, int B, int I,
                       int O, long P, int dtype);
void check_projection(const void *x, const void *Q1, const void *q1, const void *Q2, const void *q2, const void *y,
                      int B, int I, int J, int C, long P, int dtype);
void check_lift_fold(const void *P, const void *p, const void *w, const void *Wb, const void *b, const void *wf,
                     const void *af, const void *bf, int K, int J, int C, int dtype);
void check_block_rows(const void *zg, const void *zexp, const void *tb, const void *x, const void *wb,
                      const void *bias, const void *y, int B, int Ci, int Co, int H, int W, int NN, int dtype);

}  // namespace fno

#define FNO_BOUNDS(...) __VA_ARGS__

#else

#define FNO_BOUNDS(...)

#endif
