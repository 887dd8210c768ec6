// Split-K softmax attention for many query rows per KV head (d = 128, bf16):
// the exact document path at batched decode and prefill (Eq. (3.1) of the
// Nectar notes), the Quadrature module and the causal local part (section
// 2.2) when a KV head serves more than 16 query rows.
//
// A block of NW waves owns 16 * NW * RT consecutive query rows of one problem
// (KV head, and question for per-question caches) and one key range; every
// wave holds RT tiles of 16 rows (NW = 8 puts two waves on each SIMD, so one
// wave's softmax overlaps the other's matrix work).  The block streams its keys through LDS in
// stages of kStageKeys keys (64 keys: 16 KB of K, 16 KB of V), three stages in a ring: each
// lane copies 16-byte pieces from HBM straight into LDS (global_load_lds, no
// register staging), two stages ahead of use, so every key is read from HBM
// once per block whatever the number of rows.
//
// LDS layout of a stage: one 256-byte row per key, the row's 16-byte piece j
// stored at position j ^ (key & 15).  The MFMA operand reads below (16 lanes
// reading the same piece of 16 consecutive keys, or 16 pieces of one key)
// then touch 16 distinct positions, i.e. every bank once.
//
// Per 32-key tile a wave reads its operands from LDS once and reuses them for
// its RT row tiles:
//   S^T (32 keys x 16 rows) = K_tile . Q^T    (K rows as MFMA A operands)
//   P = exp2(S * scale * log2e - m) -> bf16  (row statistics in the lane)
//   O^T (128 x 16 rows) += V_tile^T . P^T    (V transposed inside the lane)
// The running max is moved only when a score exceeds it by more than
// kSlack (log2 units): until then the old reference stays, so the O rescale is
// skipped; P <= 2^kSlack keeps every sum finite and the result is unchanged
// (the same reference max is used for the numerator and the denominator).
// The 32-row kernel tests the weights instead of the scores: it exponentiates a
// tile against the current reference and looks for the tile's maximum only
// when the tile's weights in a lane sum past 2^kSlack (any weight above 2^kSlack
// does), so the common tile skips the max reduction.
#include "attn_common.hpp"
#include "lds_common.hpp"

namespace nectar {

namespace {

constexpr int kD = 128, kKS = 4, kDV = 8;
constexpr int kStages = 3;
constexpr int kPieces = kD * 2 / 16;            // 16-byte pieces per key row
constexpr float kSlack = 8.0f;
constexpr float kSlackSum = 256.0f;                // 2^kSlack
// Cache policy of the K/V copies: non-temporal (the cache is streamed once per
// call; measured 6 % faster on a 2 GB cache than the default policy).
constexpr int kStreamPolicy = 2;

}  // namespace

// Sum of a lane's 16 tile weights as a balanced tree (four dependent adds).
__device__ __forceinline__ float tile_sum16(const float (&p)[16]) {
    float s8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) s8[j] = p[2 * j] + p[2 * j + 1];
#pragma unroll
    for (int j = 0; j < 4; ++j) s8[j] += s8[j + 4];
    return (s8[0] + s8[2]) + (s8[1] + s8[3]);
}

// The kernel body for block `bid` of problem set `a` (shared by the launch of one
// set and the launch of two sets side by side).
template <int NW, int RT, int kStageKeys>
__device__ __forceinline__ void attn_rows_lds_body(const AttnParams &a, unsigned bid) {
    constexpr int kKeysPerWave = kStageKeys / NW;       // keys of a stage one wave copies
    constexpr int kCopies = kKeysPerWave / 4;           // copy instructions per wave, K and V each
    static_assert(kCopies >= 1 && kCopies * 4 * NW == kStageKeys, "stage split");
    // Three stage buffers, [0: K, 1: V][key * 16 + position].  They are
    // separate variables (not one indexed array) so the compiler can tell the
    // copies into one buffer from reads of another and does not make every
    // read wait for all copies in flight.
    __shared__ u32x4 kv_a[2][kStageKeys * kPieces], kv_b[2][kStageKeys * kPieces], kv_c[2][kStageKeys * kPieces];

    const int t = threadIdx.x, w = t >> 6, lane = t & 63, g = lane >> 4, c = lane & 15;
    // Block -> (problem p, key split sb, row block rb).  Row blocks of one
    // (p, sb) read the same keys; with xcd_group they are placed 8 ids apart,
    // which the dispatcher sends to the same XCD (ids go round-robin over the
    // 8 XCDs), so the second read of each stage hits that XCD's L2.
    int u, rb;
    if (a.xcd_group) {
        const int x = bid & 7, y = bid >> 3;
        rb = y % a.RB;
        u = (y / a.RB) * 8 + x;
    } else {
        u = bid / a.RB;
        rb = bid - u * a.RB;
    }
    const int p = u / a.SB, sb = u - p * a.SB;
    const int b = p / a.Hkv, h = p - b * a.Hkv;
    const uint16_t *kb = (const uint16_t *)a.k + b * a.kv_bstride + h * a.kv_hstride;
    const uint16_t *vb = (const uint16_t *)a.v + b * a.kv_bstride + h * a.kv_hstride;
    constexpr int kBlockRows = 16 * NW * RT;

    u32x4 qv[RT][kKS];
    int lim[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int rho = rb * kBlockRows + (w * RT + rt) * 16 + c;
        if (rho < a.Rp) {
            const int tk = rho / a.G, gg = rho - tk * a.G;
            const uint16_t *qp = (const uint16_t *)a.q + ((size_t)(b * a.Tq + tk) * a.Hq + h * a.G + gg) * kD;
#pragma unroll
            for (int kt = 0; kt < kKS; ++kt) qv[rt][kt] = *(const u32x4 *)(qp + (4 * kt + g) * 8);
            int L = a.T_kv;
            if (a.causal) L = min(L, a.q_offset + tk + 1);
            lim[rt] = max(L, 0);
        } else {
#pragma unroll
            for (int kt = 0; kt < kKS; ++kt) qv[rt][kt] = u32x4{0u, 0u, 0u, 0u};
            lim[rt] = 0x7fffffff;      // row past the end: computed unmasked, never written
        }
    }
    // Scores are formed unscaled and the scale enters the exponent's FMA; a
    // negative scale is carried by the query's sign (exact for bf16).
    float sl2 = a.sl2;
    if (sl2 < 0.f) {
        sl2 = -sl2;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int kt = 0; kt < kKS; ++kt) qv[rt][kt] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
    }

    // Key limit of the whole block (uniform): the causal limit grows with the
    // token, so the block's last valid row has the largest one.
    int blim = a.T_kv;
    if (a.causal) {
        const int last = min(a.Rp, (rb + 1) * kBlockRows) - 1;
        blim = min(blim, a.q_offset + last / a.G + 1);
    }
    blim = max(blim, 0);
    const int k_lo = sb * a.chunk;
    const int k_hi = min(k_lo + a.chunk, blim);
    const int nst = k_hi > k_lo ? (k_hi - k_lo + kStageKeys - 1) / kStageKeys : 0;
    const int kmax = a.T_kv - 1;

    // Stage i: wave w copies its kKeysPerWave keys of K and of V, four keys
    // (1 KB of LDS, lane order) per instruction; lane l fills position l & 15
    // of key r = kKeysPerWave * w + 4u + (l >> 4) with that key's piece
    // (l & 15) ^ (r & 15).
    auto issue = [&](int i, u32x4 (&dst)[2][kStageKeys * kPieces]) {
        const int key0 = k_lo + i * kStageKeys;
#pragma unroll
        for (int u = 0; u < kCopies; ++u) {
            const int r0 = kKeysPerWave * w + 4 * u, r = r0 + (lane >> 4);
            const int key = min(key0 + r, kmax);
            const int piece = (lane & 15) ^ (r & 15);
            const size_t off = (size_t)key * a.kv_row + piece * 8;
            __builtin_amdgcn_global_load_lds((const void *)(kb + off), (lds_void *)&dst[0][r0 * kPieces],
                                             16, 0, kStreamPolicy);
            __builtin_amdgcn_global_load_lds((const void *)(vb + off), (lds_void *)&dst[1][r0 * kPieces],
                                             16, 0, kStreamPolicy);
        }
    };

    f32x4 O[RT][kDV];
    float m[RT], l[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        m[rt] = -INFINITY;
        l[rt] = 0.f;
#pragma unroll
        for (int mm = 0; mm < kDV; ++mm) O[rt][mm] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // Stage i is read from buffer i % 3; its copies are issued while stage
    // i - 2 is computed (two stages ahead).
    auto step = [&](int i, const u32x4 (&cur)[2][kStageKeys * kPieces], u32x4 (&ahead)[2][kStageKeys * kPieces]) {
        // stage i has landed once at most the next stage's copies are pending
        if (i + 1 < nst) wait_vmcnt<2 * kCopies>();
        else wait_vmcnt<0>();
        stage_barrier();
        if (i + 2 < nst) issue(i + 2, ahead);
        const u32x4 *Ks = cur[0];
        const u32x4 *Vs = cur[1];
#pragma unroll
        for (int sub = 0; sub < kStageKeys / 32; ++sub) {
            const int kbase = k_lo + i * kStageKeys + 32 * sub;
            u32x4 kop[2][kKS];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int r = 32 * sub + 16 * hh + c;
#pragma unroll
                for (int kt = 0; kt < kKS; ++kt) kop[hh][kt] = Ks[r * kPieces + ((4 * kt + g) ^ c)];
            }
            u32x4 vr[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int r = 32 * sub + slot_key(g, j);
                vr[j] = Vs[r * kPieces + (c ^ (r & 15))];
            }
            // vt[mm] slot j = V[key(g, j)][8c + mm]
            u32x4 vt[kDV];
#pragma unroll
            for (int mm = 0; mm < kDV; ++mm) {
#pragma unroll
                for (int q2 = 0; q2 < 4; ++q2) {
                    // low or high halves of two keys' words: (a0 & 0xffff) | (a1 << 16)
                    // or (a0 >> 16) | (a1 & 0xffff0000), one byte permute
                    vt[mm][q2] = __builtin_amdgcn_perm(vr[2 * q2 + 1][mm >> 1], vr[2 * q2][mm >> 1],
                                                       (mm & 1) ? 0x07060302u : 0x05040100u);
                }
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kt = 0; kt < kKS; ++kt) {
                    s0 = mfma16(kop[0][kt], qv[rt][kt], s0);
                    s1 = mfma16(kop[1][kt], qv[rt][kt], s1);
                }
                float sv[8];
#pragma unroll
                for (int r = 0; r < 4; ++r) { sv[r] = s0[r]; sv[4 + r] = s1[r]; }
                // per-lane test: the compiler turns it into selects that it can
                // schedule with the matrix work (a wave-uniform branch here
                // splits the block and measured slower)
                if (kbase + 32 > lim[rt]) {
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        if (kbase + slot_key(g, j) >= lim[rt]) sv[j] = -INFINITY;
                }
                const float mt = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                                       fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7]))) * sl2;
                // move the reference max only when some score passes it by kSlack
                if (__ballot(mt > m[rt] + kSlack) != 0) {
                    const float mnew = fmaxf(m[rt], group4_max(mt));
                    const float sc = (m[rt] == -INFINITY) ? 0.f : fast_exp2(m[rt] - mnew);
                    l[rt] *= sc;
#pragma unroll
                    for (int mm = 0; mm < kDV; ++mm) O[rt][mm] *= sc;
                    m[rt] = mnew;
                }
                const float nm = (m[rt] == -INFINITY) ? 0.f : -m[rt];
                float pv[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    pv[j] = fast_exp2(__builtin_fmaf(sv[j], sl2, nm));
                    l[rt] += pv[j];
                }
                const u32x4 P = {pack_bf16(pv[0], pv[1]), pack_bf16(pv[2], pv[3]), pack_bf16(pv[4], pv[5]),
                                 pack_bf16(pv[6], pv[7])};
#pragma unroll
                for (int mm = 0; mm < kDV; ++mm) O[rt][mm] = mfma16(vt[mm], P, O[rt][mm]);
            }
        }
    };
    if (nst > 0) issue(0, kv_a);
    if (nst > 1) issue(1, kv_b);
    for (int i = 0; i < nst; i += kStages) {
        step(i, kv_a, kv_c);
        if (i + 1 >= nst) break;
        step(i + 1, kv_b, kv_a);
        if (i + 2 >= nst) break;
        step(i + 2, kv_c, kv_b);
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) l[rt] = group4_sum(l[rt]);

#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int rho = rb * kBlockRows + (w * RT + rt) * 16 + c;
        if (rho >= a.Rp) continue;
        if (a.SB == 1 && !a.defer) {
            finish_row_lanes<kD, uint16_t>(a, out_row(p, rho, a.Hkv, a.G, a.Tq, a.Hq), g, m[rt], l[rt], O[rt]);
        } else {
            const size_t row = (size_t)(p * a.SB + sb) * a.Rp + rho;
            if (g == 0) a.part_ml[row] = make_float2(m[rt], l[rt]);
            float *op = a.part_O + row * kD;
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int m4 = 0; m4 < kDV; m4 += 4) {
                    f32x4 v = {O[rt][m4][r], O[rt][m4 + 1][r], O[rt][m4 + 2][r], O[rt][m4 + 3][r]};
                    *(f32x4 *)(op + kDV * (4 * g + r) + m4) = v;
                }
        }
    }
}

template <int NW, int RT, int kStageKeys>
__global__ __launch_bounds__(NW * 64, (lds_blocks_per_cu(kStageKeys))) void attn_rows_lds(AttnParams a) {
    attn_rows_lds_body<NW, RT, kStageKeys>(a, blockIdx.x);
}

// Two problem sets in one grid, the first set's blocks first (the Quadrature
// pairs beside the decode local part: the local blocks run beside the pairs'
// instead of in a launch of their own).  Neither set may use xcd_group.
template <int NW, int RT, int kStageKeys>
__global__ __launch_bounds__(NW * 64, (lds_blocks_per_cu(kStageKeys))) void attn_rows_lds_pair(AttnGroup gr) {
    const unsigned b = blockIdx.x;
    const bool second = b >= (unsigned)gr.nb0;
    const AttnParams &a = second ? gr.p[1] : gr.p[0];
    attn_rows_lds_body<NW, RT, kStageKeys>(a, second ? b - (unsigned)gr.nb0 : b);
}

// ---------------------------------------------------------------------------
// 32 rows per wave: the same LDS ring with v_mfma_f32_32x32x16_bf16, so every
// K and V operand read from LDS serves 32 query rows (twice the 16-row kernel
// above), and a block of eight waves covers 256 rows.
//
// Per 32-key tile:
//   S^T (32 keys x 32 rows) = sum over 8 slices of 16 dims of K_slice . Q^T_slice
//       (lane l reads 16 bytes of key l % 32 in its half's 8 dims);
//   row statistics: a lane holds 16 of its row's 32 scores, the other 16 sit
//       in lane l ^ 32, so the row max and sum need one cross-lane step;
//   O^T (128 dims x 32 rows) += V^T . P^T as 4 dim blocks x 2 key groups.
// The accumulator layout of S puts key 8 (i / 4) + 4 h + i % 4 in register i of
// a lane of half h; the P^T operand of key group t is simply registers
// 8t .. 8t + 7 of that lane, provided the contraction slots of the V^T operand
// follow the same key order: slot s of half h is key 16 t + 8 (s / 4) + 4 h + s % 4.
// Those operands come straight from the key-major V stage by gfx950's
// transposing LDS read (ds_read_b64_tr_b16, four keys' values of one dim per
// lane and read; no register permutes): O^T row m of block mi is dim 32 mi + m.
// This kernel's V stages place piece j of key r at position j ^ tr_swizzle(r),
// so those reads are conflict-free too (K stages keep j ^ (r & 15)).  The
// batch-64 decode layer's document pass: 369 -> 352 us.
template <int NW, int kStageKeys>
__global__ __launch_bounds__(NW * 64, 1) void attn_rows_lds32(AttnParams a) {
    constexpr int kKeysPerWave = kStageKeys / NW;
    constexpr int kCopies = kKeysPerWave / 4;
    static_assert(kCopies >= 1 && kCopies * 4 * NW == kStageKeys, "stage split");
    constexpr int kBlockRows = 32 * NW;
    __shared__ u32x4 kv_a[2][kStageKeys * kPieces], kv_b[2][kStageKeys * kPieces], kv_c[2][kStageKeys * kPieces];

    const int t = threadIdx.x, w = t >> 6, lane = t & 63, hf = lane >> 5, r = lane & 31;
    int u, rb;
    if (a.xcd_group) {
        const int x = blockIdx.x & 7, y = blockIdx.x >> 3;
        rb = y % a.RB;
        u = (y / a.RB) * 8 + x;
    } else {
        u = blockIdx.x / a.RB;
        rb = blockIdx.x - u * a.RB;
    }
    const int p = u / a.SB, sb = u - p * a.SB;
    const int b = p / a.Hkv, h = p - b * a.Hkv;
    const uint16_t *kb = (const uint16_t *)a.k + b * a.kv_bstride + h * a.kv_hstride;
    const uint16_t *vb = (const uint16_t *)a.v + b * a.kv_bstride + h * a.kv_hstride;

    // this lane's query row and its 8 B operands (dims 16 kt + 8 hf .. + 7)
    const int rho = rb * kBlockRows + w * 32 + r;
    u32x4 qv[8];
    int lim;
    if (rho < a.Rp) {
        const int tk = rho / a.G, gg = rho - tk * a.G;
        const uint16_t *qp = (const uint16_t *)a.q + ((size_t)(b * a.Tq + tk) * a.Hq + h * a.G + gg) * kD;
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) qv[kt] = *(const u32x4 *)(qp + 16 * kt + 8 * hf);
        int L = a.T_kv;
        if (a.causal) L = min(L, a.q_offset + tk + 1);
        lim = max(L, 0);
    } else {
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) qv[kt] = u32x4{0u, 0u, 0u, 0u};
        lim = 0x7fffffff;
    }
    float sl2 = a.sl2;
    if (sl2 < 0.f) {
        sl2 = -sl2;
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) qv[kt] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
    }
    int blim = a.T_kv;
    if (a.causal) {
        const int last = min(a.Rp, (rb + 1) * kBlockRows) - 1;
        blim = min(blim, a.q_offset + last / a.G + 1);
    }
    blim = max(blim, 0);
    const int k_lo = sb * a.chunk;
    const int k_hi = min(k_lo + a.chunk, blim);
    const int nst = k_hi > k_lo ? (k_hi - k_lo + kStageKeys - 1) / kStageKeys : 0;
    const int kmax = a.T_kv - 1;

    auto issue = [&](int i, u32x4 (&dst)[2][kStageKeys * kPieces]) {
        const int key0 = k_lo + i * kStageKeys;
#pragma unroll
        for (int c = 0; c < kCopies; ++c) {
            const int r0 = kKeysPerWave * w + 4 * c, rr = r0 + (lane >> 4);
            const int key = min(key0 + rr, kmax);
            // K rows swizzled by the key (conflict-free 16-byte reads), V rows by
            // tr_swizzle (conflict-free transposing reads)
            const size_t row = (size_t)key * a.kv_row;
            const int kpiece = (lane & 15) ^ (rr & 15), vpiece = (lane & 15) ^ tr_swizzle(rr);
            __builtin_amdgcn_global_load_lds((const void *)(kb + row + kpiece * 8), (lds_void *)&dst[0][r0 * kPieces], 16, 0, kStreamPolicy);
            __builtin_amdgcn_global_load_lds((const void *)(vb + row + vpiece * 8), (lds_void *)&dst[1][r0 * kPieces], 16, 0, kStreamPolicy);
        }
    };

    // Byte offsets, within a 16-key block of a V stage, of the 8-byte slot this
    // lane names for the transposing read of key half `hh` and dim block mi:
    // key 8 hh + 4 (lane / 32) + (lane / 4) % 4, dims 32 mi + 16 ((lane / 16) % 2)
    // + 4 (lane % 4) .. + 3 (their 16-byte piece at its tr_swizzle position).
    // Lane 32 h + m then receives dim 32 mi + m of keys 8 hh + 4 h + 0..3, the
    // contraction order of the P^T operand.
    uint32_t voff[2][4];
    {
        const int G = lane >> 4, aa = lane & 3, e = (lane >> 2) & 3;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                const int key = 8 * hh + 4 * (G >> 1) + e;
                const int piece = 4 * mi + 2 * (G & 1) + (aa >> 1);
                voff[hh][mi] = (uint32_t)(key * kPieces * 16 + ((piece ^ tr_swizzle(key)) * 16) + (aa & 1) * 8);
            }
    }

    f32x16 O[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) O[mi] = f32x16{};
    float m = -INFINITY, l = 0.f;

    auto step = [&](int i, const u32x4 (&cur)[2][kStageKeys * kPieces], u32x4 (&ahead)[2][kStageKeys * kPieces]) {
        if (i + 1 < nst) wait_vmcnt<2 * kCopies>();
        else wait_vmcnt<0>();
        stage_barrier();
        if (i + 2 < nst) issue(i + 2, ahead);
        const u32x4 *Ks = cur[0];
        const u32x4 *Vs = cur[1];
#pragma unroll
        for (int sub = 0; sub < kStageKeys / 32; ++sub) {
            const int kbase = k_lo + i * kStageKeys + 32 * sub;
            f32x16 S = {};
            const int kr = 32 * sub + r;                 // the key whose 16-dim slices this lane supplies
#pragma unroll
            for (int kt = 0; kt < 8; ++kt) S = mfma32(Ks[kr * kPieces + ((2 * kt + hf) ^ (kr & 15))], qv[kt], S);
            float sv[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) sv[j] = S[j];
            if (kbase + 32 > lim) {
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    if (kbase + 8 * (j >> 2) + 4 * hf + (j & 3) >= lim) sv[j] = -INFINITY;
            }
            // weights against the current reference first; the tile's maximum is
            // looked for only when they sum past 2^kSlack (some weight above
            // 2^(kSlack - 4)) or the row has no reference yet and a key of the
            // tile is visible to it (a row masked to nothing keeps none)
            float nm = (m == -INFINITY) ? 0.f : -m;
            float pv[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) pv[j] = fast_exp2(__builtin_fmaf(sv[j], sl2, nm));
            float lt = tile_sum16(pv);
            if (__ballot((m == -INFINITY && kbase < lim) || !(lt <= kSlackSum)) != 0) {
                float mt = sv[0];
#pragma unroll
                for (int j = 1; j < 16; ++j) mt = fmaxf(mt, sv[j]);
                mt *= sl2;
                const float mnew = fmaxf(m, fmaxf(mt, __shfl_xor(mt, 32, 64)));
                const float sc = (m == -INFINITY) ? 0.f : fast_exp2(m - mnew);
                l *= sc;
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) O[mi] *= sc;
                m = mnew;
                nm = (m == -INFINITY) ? 0.f : -m;
#pragma unroll
                for (int j = 0; j < 16; ++j) pv[j] = fast_exp2(__builtin_fmaf(sv[j], sl2, nm));
                lt = tile_sum16(pv);
            }
            l += lt;
#pragma unroll
            for (int tg = 0; tg < 2; ++tg) {
                const u32x4 P = {pack_bf16(pv[8 * tg + 0], pv[8 * tg + 1]), pack_bf16(pv[8 * tg + 2], pv[8 * tg + 3]),
                                 pack_bf16(pv[8 * tg + 4], pv[8 * tg + 5]), pack_bf16(pv[8 * tg + 6], pv[8 * tg + 7])};
                // V^T operand of dim block mi, straight from LDS by transposing reads
                const char *vblk = (const char *)Vs + (32 * sub + 16 * tg) * (kPieces * 16);
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) {
                    const u32x2 h0 = lds_read_tr16(vblk, voff[0][mi]), h1 = lds_read_tr16(vblk, voff[1][mi]);
                    O[mi] = mfma32(u32x4{h0.x, h0.y, h1.x, h1.y}, P, O[mi]);
                }
            }
        }
    };
    if (nst > 0) issue(0, kv_a);
    if (nst > 1) issue(1, kv_b);
    for (int i = 0; i < nst; i += kStages) {
        step(i, kv_a, kv_c);
        if (i + 1 >= nst) break;
        step(i + 1, kv_b, kv_a);
        if (i + 2 >= nst) break;
        step(i + 2, kv_c, kv_b);
    }
    l += __shfl_xor(l, 32, 64);
    if (rho >= a.Rp) return;

    // registers 4q .. 4q + 3 of block mi hold dims 32 mi + 8 q + 4 hf + 0..3
    const bool empty = (m == -INFINITY);
    if (a.SB == 1 && !a.defer) {
        const size_t o = out_row(p, rho, a.Hkv, a.G, a.Tq, a.Hq);
        const float inv = empty ? 0.f : 1.0f / l;
        if (a.lse_out && hf == 0) a.lse_out[o] = empty ? -INFINITY : (m + log2f(l)) * kLn2;
        float wl = 0.f, wx = 0.f, it = 0.f;
        bool none = true;
        if (a.x_lse) {
            const float mx = a.x_lse[o] * kLog2e;
            const float Mt = fmaxf(m, mx);
            none = (Mt == -INFINITY);
            wl = (none || empty) ? 0.f : exp2f(m - Mt);
            wx = none ? 0.f : exp2f(mx - Mt);
            const float Lt = wl * l + wx;
            it = none ? 0.f : 1.0f / Lt;
            if (a.out_lse && hf == 0) a.out_lse[o] = none ? -INFINITY : (Mt + log2f(Lt)) * kLn2;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int mi = i >> 2, q = i & 3;
            const int dc = 32 * mi + 8 * q + 4 * hf;
            const f32x4 v = {O[mi][4 * q], O[mi][4 * q + 1], O[mi][4 * q + 2], O[mi][4 * q + 3]};
            if (a.A_out) *(f32x4 *)(a.A_out + o * kD + dc) = v * inv;
            if (a.x_lse && a.out) {
                const f32x4 xa = *(const f32x4 *)(a.x_A + o * kD + dc);
                const f32x4 ov = (wl * v + wx * xa) * it;
#pragma unroll
                for (int e = 0; e < 4; ++e) st_out<uint16_t>((uint16_t *)a.out, o * kD + dc + e, none ? 0.f : ov[e]);
            }
        }
    } else {
        const size_t row = (size_t)(p * a.SB + sb) * a.Rp + rho;
        if (hf == 0) a.part_ml[row] = make_float2(m, l);
        float *op = a.part_O + row * kD;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int mi = i >> 2, q = i & 3;
            *(f32x4 *)(op + 32 * mi + 8 * q + 4 * hf) = f32x4{O[mi][4 * q], O[mi][4 * q + 1], O[mi][4 * q + 2], O[mi][4 * q + 3]};
        }
    }
}

// One wave per SIMD with 96-key stages (144 KB of LDS, two stages in flight)
// when a block's four row tiles cover the problem; otherwise the 32-row kernel
// (eight waves, two per SIMD, 64-key stages).
// RT == 2 selects the 32-row kernel (eight waves, 256 rows per block).
// Up to 64 rows per problem: four 16-row waves and 32-key stages, two blocks
// per CU (1M-token decode layer's document pass, 56 rows per KV head: 0.726 ->
// 0.80 of HBM against 96-key stages at one block per CU); more rows: the
// 32-row kernel with 64-key stages.
LdsShape lds_shape_for(int Rp) {
    return Rp <= 64 ? LdsShape{4, 1, 32, lds_blocks_per_cu(32)} : LdsShape{8, 2, 64, lds_blocks_per_cu(64)};
}

hipError_t launch_attn_rows_lds_pair(const AttnParams &p0, const AttnParams &p1, LdsShape sh, hipStream_t st) {
    if (p0.xcd_group || p1.xcd_group) return hipErrorInvalidValue;
    AttnGroup gr;
    gr.p[0] = p0;
    gr.p[1] = p1;
    gr.nb0 = (int)((long)p0.P * p0.RB * p0.SB);
    dim3 grid((unsigned)(gr.nb0 + (long)p1.P * p1.RB * p1.SB)), block(sh.NW * 64);
    if (sh.NW == 4 && sh.RT == 1 && sh.SK == 96) hipLaunchKernelGGL((attn_rows_lds_pair<4, 1, 96>), grid, block, 0, st, gr);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_attn_rows_lds(const AttnParams &p, LdsShape sh, hipStream_t st) {
    dim3 grid((unsigned)((long)p.P * p.RB * p.SB)), block(sh.NW * 64);
    if (sh.NW == 4 && sh.RT == 1 && sh.SK == 32) hipLaunchKernelGGL((attn_rows_lds<4, 1, 32>), grid, block, 0, st, p);
    else if (sh.NW == 4 && sh.RT == 1 && sh.SK == 96) hipLaunchKernelGGL((attn_rows_lds<4, 1, 96>), grid, block, 0, st, p);
    else if (sh.NW == 8 && sh.RT == 2 && sh.SK == 64) hipLaunchKernelGGL((attn_rows_lds32<8, 64>), grid, block, 0, st, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace nectar
