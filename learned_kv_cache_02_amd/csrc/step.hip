// One launch for the independent partial passes of a decode layer step: the
// register-direct attention blocks (document and/or local problem sets) and the
// MLP module's blocks side by side in one grid, so the module's short,
// latency-bound stream overlaps the document's bandwidth-bound one instead of
// following it.  Each block runs exactly one of the two bodies; both bodies are
// the ones of the standalone kernels (attn_body.hpp, mlp_body.hpp); the module
// blocks load one weight tile at a time beside the document so the kernel fits
// the attention's two waves per SIMD.
#include "attn_body.hpp"
#include "mlp_body.hpp"

namespace nectar {

// NBUF, WPS: the module blocks' weight tiles in registers and the waves per
// SIMD the kernel is built for -- (1, two) beside the document's blocks; three
// tiles at one wave per SIMD when only the short local part shares the launch
// (4B Nectar path 15.9 -> 15.45 us; two tiles 15.56, four 15.59 us).
constexpr int kStepMlpTiles = 3;
template <int D, int ACT, int NBUF, int WPS>
__global__ __launch_bounds__(256, WPS) void step_partials(AttnGroup gr, int nb_attn, MlpParams m) {
    const int b = (int)blockIdx.x;
    if (b < nb_attn) {
        const int set = group_set(gr, b);
        attn_partial_body<D, 1, NECTAR_RT1_SUB, uint16_t>(gr.p[set], b - (set ? gr.nb0 : 0));
    } else {
        mlp_partial_body<D, 1, ACT, NBUF>(m, b - nb_attn);
    }
}

hipError_t launch_step_partials(const AttnParams &p0, const AttnParams *p1, const MlpParams &m, int d,
                                hipStream_t st) {
    AttnGroup gr;
    gr.p[0] = p0;
    gr.p[1] = p1 ? *p1 : p0;
    gr.nb0 = (int)((long)p0.P * p0.RB * p0.SB);
    const long nb_attn = gr.nb0 + (p1 ? (long)p1->P * p1->RB * p1->SB : 0);
    const long blocks = nb_attn + (long)m.Hkv * m.RB * m.SB;
    dim3 grid((unsigned)blocks), block(256);
    // a second problem set is the document: the module then runs beside a
    // bandwidth-bound stream that needs two waves per SIMD
    const bool shared = p1 != nullptr;
#define NECTAR_STEP_CASE(DD, AA) \
    if (d == DD && m.act == AA) { \
        if (shared) hipLaunchKernelGGL((step_partials<DD, AA, 1, NECTAR_RT1_WAVES_PER_SIMD>), grid, block, 0, st, gr, (int)nb_attn, m); \
        else hipLaunchKernelGGL((step_partials<DD, AA, kStepMlpTiles, 1>), grid, block, 0, st, gr, (int)nb_attn, m); \
        return hipGetLastError(); }
    NECTAR_STEP_CASE(128, 0) NECTAR_STEP_CASE(128, 1) NECTAR_STEP_CASE(128, 2)
    NECTAR_STEP_CASE(64, 0) NECTAR_STEP_CASE(64, 1) NECTAR_STEP_CASE(64, 2)
#undef NECTAR_STEP_CASE
    return hipErrorInvalidValue;
}

}  // namespace nectar
