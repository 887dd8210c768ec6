// Deep MLP module with input re-injection, Eq. (3.6) of the Nectar notes
// (section 2.4): every layer of a network reads the query again beside the
// previous layer's state, h_{k+1} = act(V_k q + U_k h_k + b_k), and each head
// ends in a linear read-out of its last state.  A layer is one contraction
// over the concatenated input [q | h_k] for all rows of all KV heads; layers
// run as consecutive launches (each needs the whole previous state), the score
// and target heads of one depth side by side in one launch.
//
// bf16: a block owns 16 rows x 16 outputs of one KV head.  Its four waves split
// the contraction into four contiguous ranges of 32-wide steps; lane (g, c)
// loads 16 bytes of weight row n0 + c and of input row rho0 + c at offset 8 g
// of each step (the 16x16x32 MFMA operand layout, both operands straight from
// their row-major arrays), the four partial tiles are folded in LDS in a fixed
// order, and wave 0 adds the bias, applies the activation and stores the tile:
// hidden states as bf16 (round to nearest even), read-outs as fp32.
// fp32: one thread per output, a plain sequential dot product.
#include "attn_common.hpp"

namespace nectar {

namespace {

__device__ __forceinline__ DeepLayer pick_layer(const DeepParams &a, long &blk) {
    if (a.nl > 1 && blk >= a.L0.blocks) {
        blk -= a.L0.blocks;
        return a.L1;
    }
    return a.L0;
}

}  // namespace

template <int D>
__global__ __launch_bounds__(256) void deep_layer_mfma(DeepParams a) {
    long blk = blockIdx.x;
    const DeepLayer L = pick_layer(a, blk);
    const int NT = (L.N + 15) / 16, RT = (a.Rp + 15) / 16;
    // output tiles fastest: blocks sharing a weight tile are NT ids apart
    const int nt = (int)(blk % NT);
    const long rest = blk / NT;
    const int rt = (int)(rest % RT), p = (int)(rest / RT);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
    const int n0 = nt * 16, rho0 = rt * 16;
    const int nl = min(n0 + c, L.N - 1), rl = min(rho0 + c, a.Rp - 1);   // loads stay in bounds
    const int Dq = L.Wq ? D : 0;
    const int steps = (Dq + L.Kh) / 32;
    const int s0 = wave * steps / 4, s1 = (wave + 1) * steps / 4;

    const uint16_t *wq = (const uint16_t *)L.Wq + ((size_t)p * L.N + nl) * D + 8 * g;
    const uint16_t *xq = (const uint16_t *)a.q + out_row(p, rl, a.Hkv, a.G, 0, a.Hq) * D + 8 * g;
    const uint16_t *wh = (const uint16_t *)L.Wh + ((size_t)p * L.N + nl) * L.Kh + 8 * g;
    const uint16_t *xh = (const uint16_t *)L.X + ((size_t)p * a.Rp + rl) * L.Kh + 8 * g;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = s0; s < s1; s += 4) {
        u32x4 wa[4], xb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int k = (s + u) * 32;
            wa[u] = u32x4{0u, 0u, 0u, 0u};
            xb[u] = u32x4{0u, 0u, 0u, 0u};
            if (s + u < s1) {
                if (k < Dq) {
                    wa[u] = *(const u32x4 *)(wq + k);
                    xb[u] = *(const u32x4 *)(xq + k);
                } else {
                    wa[u] = *(const u32x4 *)(wh + (k - Dq));
                    xb[u] = *(const u32x4 *)(xh + (k - Dq));
                }
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) acc = mfma16(wa[u], xb[u], acc);
    }

    __shared__ f32x4 red[3][64];
    if (wave > 0) red[wave - 1][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    acc += red[0][lane];
    acc += red[1][lane];
    acc += red[2][lane];

    // lane (g, c): outputs n0 + 4 g + r of row rho0 + c
    const int rho = rho0 + c;
    if (rho >= a.Rp) return;
    float y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int n = n0 + 4 * g + r;
        y[r] = acc[r] + (n < L.N ? L.b[(size_t)p * L.N + n] : 0.f);
        if (L.act >= 0) y[r] = activation(L.act, y[r]);
    }
    if (L.Y) {
        // hidden widths are multiples of 32: the four outputs are in range
        uint16_t *dst = (uint16_t *)L.Y + ((size_t)p * a.Rp + rho) * L.N + n0 + 4 * g;
        *(u32x2 *)dst = u32x2{pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])};
    } else {
        const size_t o = out_row(p, rho, a.Hkv, a.G, 0, a.Hq);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int n = n0 + 4 * g + r;
            if (n < L.N) L.Yf[o * L.N + n] = y[r];
        }
    }
}

template <int D>
__global__ __launch_bounds__(256) void deep_layer_valu(DeepParams a) {
    long blk = blockIdx.x;
    const DeepLayer L = pick_layer(a, blk);
    const long idx = blk * 256 + threadIdx.x;
    if (idx >= (long)a.Hkv * a.Rp * L.N) return;
    const int n = (int)(idx % L.N);
    const long pr = idx / L.N;
    const int rho = (int)(pr % a.Rp), p = (int)(pr / a.Rp);
    float z = L.b[(size_t)p * L.N + n];
    if (L.Wq) {
        const float *w = (const float *)L.Wq + ((size_t)p * L.N + n) * D;
        const float *x = (const float *)a.q + out_row(p, rho, a.Hkv, a.G, 0, a.Hq) * D;
        for (int k = 0; k < D; ++k) z += w[k] * x[k];
    }
    if (L.Wh) {
        const float *w = (const float *)L.Wh + ((size_t)p * L.N + n) * L.Kh;
        const float *x = (const float *)L.X + ((size_t)p * a.Rp + rho) * L.Kh;
        for (int k = 0; k < L.Kh; ++k) z += w[k] * x[k];
    }
    if (L.act >= 0) z = activation(L.act, z);
    if (L.Y) ((float *)L.Y)[((size_t)p * a.Rp + rho) * L.N + n] = z;
    else L.Yf[out_row(p, rho, a.Hkv, a.G, 0, a.Hq) * L.N + n] = z;
}

long deep_layer_blocks(int dtype, int Hkv, int Rp, int N) {
    if (dtype == 1) return (long)Hkv * ((Rp + 15) / 16) * ((N + 15) / 16);
    return ((long)Hkv * Rp * N + 255) / 256;
}

hipError_t launch_deep_layers(const DeepParams &p, int dtype, int d, hipStream_t st) {
    const long blocks = p.L0.blocks + (p.nl > 1 ? p.L1.blocks : 0);
    if (blocks <= 0) return hipSuccess;
    dim3 grid((unsigned)blocks), block(256);
    if (dtype == 1 && d == 128) hipLaunchKernelGGL(deep_layer_mfma<128>, grid, block, 0, st, p);
    else if (dtype == 1 && d == 64) hipLaunchKernelGGL(deep_layer_mfma<64>, grid, block, 0, st, p);
    else if (d == 128) hipLaunchKernelGGL(deep_layer_valu<128>, grid, block, 0, st, p);
    else if (d == 64) hipLaunchKernelGGL(deep_layer_valu<64>, grid, block, 0, st, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace nectar
