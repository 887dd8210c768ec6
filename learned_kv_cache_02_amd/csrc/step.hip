// One launch for the independent partial passes of a decode layer step: the
// register-direct attention blocks (document and/or local problem sets) and the
// MLP module's blocks side by side in one grid, so the module's short,
// latency-bound stream overlaps the document's bandwidth-bound one instead of
// following it.  Each block runs exactly one of the two bodies; both bodies are
// the ones of the standalone kernels (attn_body.hpp, mlp_body.hpp); the module
// blocks load one weight tile at a time so the kernel fits the attention's two
// waves per SIMD.
#include "attn_body.hpp"
#include "mlp_body.hpp"

namespace nectar {

template <int D, int ACT>
__global__ __launch_bounds__(256, NECTAR_RT1_WAVES_PER_SIMD) void step_partials(AttnGroup gr, int nb_attn,
                                                                                 MlpParams m) {
    const int b = (int)blockIdx.x;
    if (b < nb_attn) {
        const int set = group_set(gr, b);
        attn_partial_body<D, 1, NECTAR_RT1_SUB, uint16_t>(gr.p[set], b - (set ? gr.nb0 : 0));
    } else {
        mlp_partial_body<D, 1, ACT, false>(m, b - nb_attn);
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
#define NECTAR_STEP_CASE(DD, AA) \
    if (d == DD && m.act == AA) { hipLaunchKernelGGL((step_partials<DD, AA>), grid, block, 0, st, gr, (int)nb_attn, m); return hipGetLastError(); }
    NECTAR_STEP_CASE(128, 0) NECTAR_STEP_CASE(128, 1) NECTAR_STEP_CASE(128, 2)
    NECTAR_STEP_CASE(64, 0) NECTAR_STEP_CASE(64, 1) NECTAR_STEP_CASE(64, 2)
#undef NECTAR_STEP_CASE
    return hipErrorInvalidValue;
}

}  // namespace nectar
