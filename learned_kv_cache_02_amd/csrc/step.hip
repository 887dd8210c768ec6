// One launch for the independent partial passes of a decode layer step: the
// register-direct attention blocks (document and/or local problem sets) and the
// MLP module's blocks side by side in one grid, so the module's short,
// latency-bound stream overlaps the document's bandwidth-bound one instead of
// following it.  Each block runs exactly one of the two bodies, the ones of the
// standalone kernels: beside the document the module blocks use the
// register-direct body one weight tile at a time (mlp_body.hpp), so the kernel
// fits the attention's two waves per SIMD; beside the local part alone they use
// the decode body (mlp_decode.hpp: weights staged through LDS, up to 64 rows).
#include "attn_body.hpp"
#include "mlp_body.hpp"
#include "mlp_decode.hpp"

namespace nectar {

// Beside the document (two waves per SIMD) the module blocks run the
// register-direct body holding one weight tile at a time.
template <int D, int ACT>
__global__ __launch_bounds__(256, NECTAR_RT1_WAVES_PER_SIMD) void step_partials(AttnGroup gr, int nb_attn,
                                                                                MlpParams m) {
    const int b = (int)blockIdx.x;
    if (b < nb_attn) {
        const int set = group_set(gr, b);
        attn_partial_body<D, 1, NECTAR_RT1_SUB, uint16_t>(gr.p[set], b - (set ? gr.nb0 : 0));
    } else {
        mlp_partial_body<D, 1, ACT, 1>(m, b - nb_attn);
    }
}

// Beside the local part only: the decode module body (target and score waves,
// every tile load up front, RTM row tiles) at one wave per SIMD, or two with
// 64-row blocks at d = 128 (then the attention blocks' extra four waves end at
// once: the attention body is written for four).
template <int D, int ACT, int RTM>
__global__ __launch_bounds__((dec_threads(D, RTM)), 1) void step_partials_dec(AttnGroup gr, int nb_attn, MlpParams m) {
    // one LDS allocation for whichever body the block runs
    __shared__ union {
        DecLdsOf<D, RTM, kDecTiles> mlp;
        AttnFoldLds<D, 1> attn;
    } lds;
    const int b = (int)blockIdx.x;
    if (b < nb_attn) {
        if (threadIdx.x >= 256) return;
        const int set = group_set(gr, b);
        attn_partial_body_lds<D, 1, NECTAR_RT1_SUB, uint16_t>(gr.p[set], b - (set ? gr.nb0 : 0), lds.attn);
    } else {
        mlp_decode_body_lds<D, RTM, ACT, kDecTiles>(m, b - nb_attn, lds.mlp);
    }
}

hipError_t launch_step_partials(const AttnParams &p0, const AttnParams *p1, const MlpParams &m, int d, int mlp_rt,
                                hipStream_t st) {
    AttnGroup gr;
    gr.p[0] = p0;
    gr.p[1] = p1 ? *p1 : p0;
    gr.nb0 = (int)((long)p0.P * p0.RB * p0.SB);
    const long nb_attn = gr.nb0 + (p1 ? (long)p1->P * p1->RB * p1->SB : 0);
    const long blocks = nb_attn + (long)m.Hkv * (p1 ? m.RB : m.RG) * m.SB;
    dim3 grid((unsigned)blocks), block(256);
    // a second problem set is the document: the module then runs beside a
    // bandwidth-bound stream that needs two waves per SIMD
    const bool shared = p1 != nullptr;
#define NECTAR_STEP_CASE(DD, AA) \
    if (d == DD && m.act == AA) { \
        if (shared && mlp_rt == 1) hipLaunchKernelGGL((step_partials<DD, AA>), grid, block, 0, st, gr, (int)nb_attn, m); \
        else if (shared) return hipErrorInvalidValue; \
        else if (mlp_rt == 1) hipLaunchKernelGGL((step_partials_dec<DD, AA, 1>), grid, dim3((dec_threads(DD, 1))), 0, st, gr, (int)nb_attn, m); \
        else if (mlp_rt == 2) hipLaunchKernelGGL((step_partials_dec<DD, AA, 2>), grid, dim3((dec_threads(DD, 2))), 0, st, gr, (int)nb_attn, m); \
        else if (mlp_rt == 4) hipLaunchKernelGGL((step_partials_dec<DD, AA, 4>), grid, dim3((dec_threads(DD, 4))), 0, st, gr, (int)nb_attn, m); \
        else return hipErrorInvalidValue; \
        return hipGetLastError(); }
    NECTAR_STEP_CASE(128, 0) NECTAR_STEP_CASE(128, 1) NECTAR_STEP_CASE(128, 2)
    NECTAR_STEP_CASE(64, 0) NECTAR_STEP_CASE(64, 1) NECTAR_STEP_CASE(64, 2)
#undef NECTAR_STEP_CASE
    return hipErrorInvalidValue;
}

}  // namespace nectar
