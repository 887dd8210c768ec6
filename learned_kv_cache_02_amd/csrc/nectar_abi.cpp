// C ABI of the Nectar hot path (declared in include/nectar.h): host-side
// argument validation (before any HIP call, so every error path is testable
// without a GPU), split planning, workspace sizing and kernel dispatch.
#include "nectar.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "kernels.hpp"

// Device scratch of nectar_layer_step_static: one copy per GPU the library is
// loaded on, held until the process ends.  Host code never passes this name to
// a kernel (on the host it is only a stand-in for the symbol): it uses the
// device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[NECTAR_STATIC_SCRATCH_BYTES];

static_assert(NECTAR_MERGE_K_MAX == nectar::kMergeKMax, "K-way merge limit");

using namespace nectar;

namespace {

// Waves a split plan aims for: 256 CUs x 8 resident waves keeps every CU busy
// with enough loads in flight to cover HBM latency.
#ifndef NECTAR_TARGET_WAVES
#define NECTAR_TARGET_WAVES 2048
#endif
#ifndef NECTAR_RT1_SUB
#define NECTAR_RT1_SUB 2
#endif
constexpr long kTargetWaves = NECTAR_TARGET_WAVES;
// Weight-streaming waves a module plan aims for (decode: target plus score
// waves over all KV heads).  Fewer, longer waves stream the weights with fewer
// partials to fold: the 1M-token decode stack's Nectar path 22.5 -> 21.1 us per
// layer from 512 to 256 (with four float4 columns per finishing wave).
#ifndef NECTAR_TARGET_WAVES_MLP
#define NECTAR_TARGET_WAVES_MLP 256
#endif
constexpr long kTargetWavesMlp = NECTAR_TARGET_WAVES_MLP;
// ... when the module's blocks share one launch with the exact document's (the
// fused decode step): shorter module blocks interleave better with the
// document stream (measured: the 4B decode step 61.1 -> 59.5 us), while the
// module alone is faster with fewer, longer blocks (13.9 vs 16.1 us).
#ifndef NECTAR_TARGET_WAVES_MLP_SHARED
#define NECTAR_TARGET_WAVES_MLP_SHARED 2048
#endif
constexpr long kTargetWavesMlpShared = NECTAR_TARGET_WAVES_MLP_SHARED;
// Compute units a split plan of the LDS-staged kernel aims to fill: this many
// times the shape's blocks per CU (LdsShape::BPC, set by its LDS use).
#ifndef NECTAR_LDS_TARGET_BLOCKS
#define NECTAR_LDS_TARGET_BLOCKS 256
#endif
#ifndef NECTAR_LDS_MIN_ROWS
#define NECTAR_LDS_MIN_ROWS 17
#endif
constexpr long kTargetBlocksLds = NECTAR_LDS_TARGET_BLOCKS;
// Rows per KV head from which attention uses the LDS-staged kernel (bf16,
// d = 128): beyond one 16-row tile the register-direct kernel would stream
// the cache once per row group.
constexpr int kLdsRows = NECTAR_LDS_MIN_ROWS;
constexpr int kTile = 32;

inline long cdiv(long a, long b) { return (a + b - 1) / b; }

inline bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

nectar_status check_desc(const nectar_attn_desc *d) {
    if (!d) return NECTAR_EINVAL;
    if (d->R < 0 || d->Hq <= 0 || d->Hkv <= 0 || d->Hq % d->Hkv != 0) return NECTAR_EINVAL;
    if (d->dtype != NECTAR_F32 && d->dtype != NECTAR_BF16) return NECTAR_EINVAL;
    if (d->d <= 0) return NECTAR_EINVAL;
    if (d->d != 64 && d->d != 128) return NECTAR_EUNSUPPORTED;
    if (!std::isfinite(d->scale) || d->splits < 0) return NECTAR_EINVAL;
    // document K/V row stride: 0 (dense rows) or at least d, whole 16-byte pieces
    if (d->kv_stride != 0 && (d->kv_stride < d->d || d->kv_stride % 8 != 0 || d->kv_stride > (1 << 20)))
        return NECTAR_EINVAL;
    if ((long)d->R * d->Hq > 0x7fffffffL / 2) return NECTAR_EUNSUPPORTED;
    return NECTAR_OK;
}

inline float score_scale(const nectar_attn_desc *d) {
    return d->scale != 0.f ? d->scale : 1.0f / std::sqrt((float)d->d);
}

// Elements from one document key's K (or V) row to the next's; a KV head's
// rows start n of these apart.
inline int64_t doc_row(const nectar_attn_desc *d) { return d->kv_stride > 0 ? d->kv_stride : d->d; }

// Tensors read with 16-byte vector loads must be 16-byte aligned; fp32 scalars
// and outputs written element-wise need their natural alignment.
inline bool tensor_ok(const void *p) { return p && aligned(p, 16); }
inline bool f32_ok(const void *p) { return p && aligned(p, 4); }
// Arrays of d-vectors ([R][Hq][d] read-outs and outputs) are read and written
// with vector accesses: 16-byte aligned like every tensor.
inline bool rows_ok(const void *p) { return p && aligned(p, 16); }

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct AttnPlan {
    int P = 0, Rp = 0, RT = 0, RG = 0, S = 0, chunk = kTile, tiles = 0;
    int WR = 1, WS = 1, RB = 0, SB = 0;
    bool lds = false, xcd = false;
    LdsShape sh{0, 0, 0};
    size_t ws = 0;
};

// Block shape of the MFMA kernels: 4 waves as WR row groups x WS splits.
void block_shape(int RG, int &WR, int &WS, int &RB) {
    WR = RG >= 3 ? 4 : (RG == 2 ? 2 : 1);
    WS = 4 / WR;
    RB = (int)cdiv(RG, WR);
}

// balanced: the register-direct kernel's S splits cover floor or ceil(tiles / S)
// batches each (every CU gets the same share: the 4B document's 960 batches in
// 256 splits = 512 blocks, two per CU, instead of 240 splits of 4 = 480 blocks);
// otherwise every split but the last covers the same whole number of batches.
// lds_blocks > 0: the LDS-staged kernel whatever the row count, its split count
// aiming for that many blocks (a problem set sharing one launch with another).
AttnPlan plan_attn(const nectar_attn_desc *d, int P, int Rp, long T_kv, bool balanced = true,
                   long target_waves = kTargetWaves, long lds_blocks = 0, const LdsShape *lds_shape = nullptr) {
    AttnPlan pl;
    pl.P = P;
    pl.Rp = Rp;
    if (P == 0 || Rp == 0 || T_kv <= 0) return pl;    // nothing to attend: combine with S = 0
    const bool mfma = d->dtype == NECTAR_BF16;
    if (mfma && d->d == 128 && (Rp >= kLdsRows || lds_blocks > 0)) {
        // LDS-staged kernel: blocks of 16 * NW * RT rows x key splits of whole
        // SK-key stages; a block finishes its rows in place when S == 1
        pl.lds = true;
        pl.sh = lds_shape ? *lds_shape : lds_shape_for(Rp);
        pl.RT = pl.sh.RT;
        pl.WR = pl.sh.NW;
        pl.RB = (int)cdiv(Rp, 16L * pl.sh.NW * pl.sh.RT);
        pl.RG = (int)cdiv(Rp, 16L * pl.RT);
        const long stages = cdiv(T_kv, pl.sh.SK);
        const long target = lds_blocks > 0 ? lds_blocks : kTargetBlocksLds * pl.sh.BPC;
        long S = d->splits > 0 ? d->splits : cdiv(target, (long)P * pl.RB);
        S = S < 1 ? 1 : (S > stages ? stages : S);
        const long per = cdiv(stages, S);
        pl.chunk = (int)(per * pl.sh.SK);
        pl.S = pl.SB = (int)cdiv(stages, per);
        pl.xcd = pl.RB > 1 && pl.RB <= 8 && ((long)P * pl.S) % 8 == 0;
        pl.ws = pl.SB > 1 ? (size_t)P * pl.SB * Rp * ((size_t)d->d * 4 + 8) : 0;
        return pl;
    }
    // the MFMA kernel walks keys in batches of NECTAR_RT1_SUB 32-key tiles
    const long gran = mfma ? NECTAR_RT1_SUB * kTile : kTile;
    const long tiles = cdiv(T_kv, gran);
    long units;
    if (mfma) {
        pl.RT = row_tiles_for(Rp);
        pl.RG = (int)cdiv(Rp, 16L * pl.RT);
        block_shape(pl.RG, pl.WR, pl.WS, pl.RB);
        units = (long)P * pl.RG;
    } else {
        pl.RG = Rp;
        units = (long)P * Rp;
    }
    long S = d->splits > 0 ? d->splits : cdiv(target_waves, units);
    S = S < 1 ? 1 : (S > tiles ? tiles : S);
    if (mfma && balanced && d->splits <= 0) {
        pl.chunk = (int)gran;
        pl.tiles = (int)tiles;
        pl.S = (int)S;
    } else {
        const long per = cdiv(tiles, S);
        pl.chunk = (int)(per * gran);
        pl.S = (int)cdiv(tiles, per);
    }
    pl.SB = mfma ? (int)cdiv(pl.S, pl.WS) : pl.S;
    // [read-outs][statistics] of every per-block partial; none when one block
    // per row group covers all keys (MFMA path finishes rows in place)
    pl.ws = pl.SB > 1 || !mfma ? (size_t)P * pl.SB * Rp * ((size_t)d->d * 4 + 8) : 0;
    return pl;
}

struct MlpPlan {
    int Rp = 0, RT = 0, RG = 0, S = 0, ct = kTile, cs = kTile;
    int WR = 1, WS = 1, RB = 0, SB = 0;
    bool prefill = false;   // a batched kernel (LDS-staged weights)
    bool lds32 = false;     // ... the 32x32 one (unit counts multiples of 64)
    bool dec = false;       // the decode kernel (target and score waves)
    int Wt = 0, Ws = 0;     // ... its waves per (KV head, row group)
    size_t ws = 0;
};

// Rows per KV head up to which the register-direct kernel serves the module
// (bf16): one wave holds up to 64 rows (four 16-row tiles), so the weights
// stream once; beyond, the LDS-staged batched kernels (d = 128) share each
// weight tile between more rows.
constexpr int kPrefillRows = 65;
constexpr int kPrefillBlockRows = 256;
// Blocks a split plan of the batched kernel aims for (one 512-thread block per CU).
// Blocks a batched module plan aims for (256-row blocks x hidden-unit splits).
#ifndef NECTAR_PREFILL_TARGET_BLOCKS
#define NECTAR_PREFILL_TARGET_BLOCKS 256
#endif
constexpr long kTargetBlocksPrefill = NECTAR_PREFILL_TARGET_BLOCKS;

// The document pass of the exact-attention entry points (no other part shares
// its launch).  Up to 16 rows per KV head over a long document, the LDS-staged
// 16-row kernel with 32-key stages at two blocks per CU streams the cache
// faster than the register-direct kernel (4B layer's document partial pass
// 43.2 -> 41.2 us); inside the layer step the register-direct kernel stays,
// since its blocks share one launch with the local part's and the module's.
constexpr long kLdsDocKeys = 16384;
AttnPlan plan_doc(const nectar_attn_desc *d, long n) {
    const int Rp = d->R * (d->Hq / d->Hkv);
    if (d->dtype == NECTAR_BF16 && d->d == 128 && Rp > 0 && Rp < kLdsRows && n >= kLdsDocKeys && d->splits <= 0) {
        const LdsShape sh = lds_shape_for(Rp);
        return plan_attn(d, d->Hkv, Rp, n, true, kTargetWaves, kTargetBlocksLds * sh.BPC, &sh);
    }
    return plan_attn(d, d->Hkv, Rp, n);
}

MlpPlan plan_mlp(const nectar_attn_desc *d, int Ht, int Hs, long target_waves = kTargetWavesMlp,
                 bool shared = false) {
    MlpPlan pl;
    pl.Rp = d->R * (d->Hq / d->Hkv);
    if (pl.Rp == 0) return pl;
    const long tt = cdiv(Ht, kTile), ts = cdiv(Hs, kTile);
    const long tmax = tt > ts ? (tt > 1 ? tt : 1) : (ts > 1 ? ts : 1);
    if (d->dtype == NECTAR_BF16 && d->d == 128 && pl.Rp >= kPrefillRows && Ht % 64 == 0 && Hs % 64 == 0) {
        // 32x32 batched kernel: 256-row blocks x hidden-unit splits of whole 64-unit stages
        pl.prefill = pl.lds32 = true;
        pl.RB = (int)cdiv(pl.Rp, kPrefillBlockRows);
        const long gt = cdiv(Ht, 64), gs = cdiv(Hs, 64);
        const long gmax = gt > gs ? (gt > 1 ? gt : 1) : (gs > 1 ? gs : 1);
        long S = d->splits > 0 ? d->splits : cdiv(kTargetBlocksPrefill, (long)d->Hkv * pl.RB);
        S = S < 1 ? 1 : (S > gmax ? gmax : S);
        const long pt = cdiv(gt, S), ps = cdiv(gs, S);
        long Se = 1;
        if (pt > 0 && cdiv(gt, pt) > Se) Se = cdiv(gt, pt);
        if (ps > 0 && cdiv(gs, ps) > Se) Se = cdiv(gs, ps);
        pl.S = pl.SB = (int)Se;
        pl.ct = (int)(pt * 64);
        pl.cs = (int)(ps * 64);
        pl.ws = pl.SB > 1 ? (size_t)d->Hkv * pl.SB * pl.Rp * ((size_t)d->d * 4 + 4) : 0;
        return pl;
    }
    if (d->dtype == NECTAR_BF16 && d->d == 128 && pl.Rp >= kPrefillRows) {
        // batched kernel: 256-row blocks x hidden-unit splits of whole 32-unit chunks
        pl.prefill = true;
        pl.RB = (int)cdiv(pl.Rp, kPrefillBlockRows);
        long S = d->splits > 0 ? d->splits : cdiv(kTargetBlocksPrefill, (long)d->Hkv * pl.RB);
        S = S < 1 ? 1 : (S > tmax ? tmax : S);
        long pt = cdiv(tt, S), ps = cdiv(ts, S);
        long Se = 1;
        if (pt > 0 && cdiv(tt, pt) > Se) Se = cdiv(tt, pt);
        if (ps > 0 && cdiv(ts, ps) > Se) Se = cdiv(ts, ps);
        pl.S = pl.SB = (int)Se;
        pl.ct = (int)(pt * kTile);
        pl.cs = (int)(ps * kTile);
        pl.ws = pl.SB > 1 ? (size_t)d->Hkv * pl.SB * pl.Rp * ((size_t)d->d * 4 + 4) : 0;
        return pl;
    }
    const bool mfma = d->dtype == NECTAR_BF16;
    if (mfma && !shared) {
        // decode kernel: per (KV head, row group) Wt target waves and Ws score
        // waves, sized so every wave reads about the same number of bytes (a
        // target tile streams twice the bytes of a score tile) and holds at most
        // kDecTiles target or dec_score_tiles(RT) score tiles; target_waves is
        // the wave budget of the launch
        pl.dec = true;
        pl.RT = mlp_row_tiles(pl.Rp);
        pl.RG = pl.RB = (int)cdiv(pl.Rp, 16L * pl.RT);
        pl.WR = 1;
        // WS: tile slots per block, set below
        const long per = (long)d->Hkv * pl.RG;
        const long Wa = std::max(1L, d->splits > 0 ? (long)d->splits : cdiv(target_waves, per));
        auto clampl = [](long x, long lo, long hi) { return std::min(std::max(x, lo), hi); };
        const long smax = dec_score_tiles(pl.RT);   // score tiles per wave
        long Wt = 0, Ws = 0;
        if (tt > 0 && ts > 0) {
            Wt = clampl(std::lround((double)Wa * 2.0 * tt / (2.0 * tt + ts)), cdiv(tt, kDecTiles), tt);
            Ws = clampl(Wa - Wt, cdiv(ts, smax), ts);
        } else if (tt > 0) {
            Wt = clampl(Wa, cdiv(tt, kDecTiles), tt);
        } else if (ts > 0) {
            Ws = clampl(Wa, cdiv(ts, smax), ts);
        }
        pl.Wt = (int)Wt;
        pl.Ws = (int)Ws;
        pl.S = (int)(Wt + Ws);
        pl.WS = dec_slots(d->d, pl.RT);
        pl.SB = (int)std::max(1L, cdiv(Wt + Ws, (long)pl.WS));
        pl.ws = pl.SB > 1 ? (size_t)d->Hkv * pl.SB * pl.Rp * ((size_t)d->d * 4 + 4) : 0;
        return pl;
    }
    // register-direct body one tile at a time (beside the document in the fused
    // decode step; RT == 1 there) and the fp32 path: S splits of pt target and
    // ps score tiles each
    long units;
    if (mfma) {
        pl.RT = row_tiles_for(pl.Rp);
        pl.RG = (int)cdiv(pl.Rp, 16L * pl.RT);
        block_shape(pl.RG, pl.WR, pl.WS, pl.RB);
        units = (long)d->Hkv * pl.RG;
    } else {
        pl.RG = pl.Rp;
        units = (long)d->Hkv * pl.Rp;
    }
    long S = d->splits > 0 ? d->splits : cdiv(target_waves, units);
    S = S < 1 ? 1 : (S > tmax ? tmax : S);
    long pt = cdiv(tt, S), ps = cdiv(ts, S);
    pt = pt < 1 ? 1 : pt;
    ps = ps < 1 ? 1 : ps;
    long Se = cdiv(tt, pt);
    if (cdiv(ts, ps) > Se) Se = cdiv(ts, ps);
    if (Se < 1) Se = 1;
    pl.S = (int)Se;
    pl.ct = (int)(pt * kTile);
    pl.cs = (int)(ps * kTile);
    pl.SB = mfma ? (int)cdiv(pl.S, pl.WS) : pl.S;
    pl.ws = pl.SB > 1 || !mfma ? (size_t)d->Hkv * pl.SB * pl.Rp * ((size_t)d->d * 4 + 4) : 0;
    return pl;
}

nectar_status check_ws(size_t need, const void *ws, size_t ws_bytes) {
    if (need == 0) return NECTAR_OK;
    if (ws_bytes < need) return NECTAR_EWORKSPACE;
    return (ws && aligned(ws, 16)) ? NECTAR_OK : NECTAR_EINVAL;
}

nectar_status finish(hipError_t e, hipStream_t st) {
    if (e != hipSuccess) return NECTAR_EHIP;
    static const bool sync_check = [] {
        const char *v = std::getenv("NECTAR_SYNC_CHECK");
        return v && v[0] == '1';
    }();
    if (sync_check) {
        if (hipStreamSynchronize(st) != hipSuccess) return NECTAR_EHIP;
        if (hipGetLastError() != hipSuccess) return NECTAR_EHIP;
    }
    return NECTAR_OK;
}

// Attention over a batched cache, then (unless one block per row group covered
// every key) the combine pass.
hipError_t run_attention(const nectar_attn_desc *d, const AttnPlan &pl, const void *q, const void *k,
                         const void *v, int64_t bstride, int64_t hstride, int64_t row, int B, int Tq, long T_kv,
                         int causal, int q_offset, CombineParams cp, void *ws, hipStream_t st) {
    const bool mfma = d->dtype == NECTAR_BF16;
    float *part_O = (float *)ws;
    float2 *part_ml = (float2 *)((char *)part_O + (size_t)pl.P * pl.SB * pl.Rp * d->d * 4);
    if (pl.S > 0) {
        AttnParams a{};
        a.q = q; a.k = k; a.v = v;
        a.kv_bstride = bstride; a.kv_hstride = hstride; a.kv_row = row;
        a.Hq = d->Hq; a.G = d->Hq / d->Hkv; a.Hkv = d->Hkv; a.Tq = Tq; a.B = B; a.Rp = pl.Rp;
        a.T_kv = (int)T_kv; a.causal = causal; a.q_offset = q_offset;
        a.sl2 = score_scale(d) * 1.4426950408889634f;
        a.P = pl.P; a.S = pl.S; a.chunk = pl.chunk; a.tiles = pl.tiles; a.RG = pl.RG;
        a.WR = pl.WR; a.WS = pl.WS; a.RB = pl.RB; a.SB = pl.SB;
        a.xcd_group = pl.xcd ? 1 : 0;
        a.part_O = part_O; a.part_ml = part_ml;
        if (mfma && pl.SB == 1) {
            a.lse_out = cp.lse_out; a.A_out = cp.A_out; a.x_lse = cp.x_lse; a.x_A = cp.x_A;
            a.out = cp.out; a.out_lse = cp.out_lse;
        }
        hipError_t e = pl.lds ? launch_attn_rows_lds(a, pl.sh, st) : launch_attn_partial(a, d->dtype, d->d, pl.RT, st);
        if (e != hipSuccess || (mfma && pl.SB == 1)) return e;
    }
    cp.part_O = part_O; cp.part_ml = part_ml;
    cp.Hq = d->Hq; cp.G = d->Hq / d->Hkv; cp.Hkv = d->Hkv; cp.Tq = Tq;
    cp.P = pl.P; cp.S = pl.SB; cp.Rp = pl.Rp;
    return launch_attn_combine(cp, d->dtype, d->d, st);
}

}  // namespace

extern "C" {

int nectar_abi_version(void) { return NECTAR_ABI_VERSION; }

nectar_status nectar_workspace_init(void *ws, size_t ws_bytes, void *stream) {
    if (ws_bytes == 0) return NECTAR_OK;
    if (!ws || !aligned(ws, 16)) return NECTAR_EINVAL;
    hipStream_t st = (hipStream_t)stream;
    return finish(launch_fill_zero(ws, ws_bytes, st), st);
}

const char *nectar_status_string(nectar_status s) {
    switch (s) {
        case NECTAR_OK: return "NECTAR_OK: success";
        case NECTAR_EINVAL: return "NECTAR_EINVAL: invalid argument (null pointer, shape, alignment or enum)";
        case NECTAR_EUNSUPPORTED: return "NECTAR_EUNSUPPORTED: valid arguments not supported by this library";
        case NECTAR_EWORKSPACE: return "NECTAR_EWORKSPACE: workspace smaller than the size query requires";
        case NECTAR_EHIP: return "NECTAR_EHIP: HIP launch or execution error";
    }
    return "unknown nectar_status";
}

size_t nectar_doc_attn_workspace_size(const nectar_attn_desc *desc, int64_t n) {
    if (check_desc(desc) != NECTAR_OK || n < 0 || n > 0x7fffffffL - kTile) return 0;
    return plan_doc(desc, (long)n).ws;
}

nectar_status nectar_doc_attn_exact(const nectar_attn_desc *desc, int64_t n, const void *q,
                                    const void *k, const void *v, float *alpha_out, float *A_out,
                                    void *ws, size_t ws_bytes, void *stream) {
    nectar_status s = check_desc(desc);
    if (s != NECTAR_OK) return s;
    if (n < 0) return NECTAR_EINVAL;
    if (n > 0x7fffffffL - kTile) return NECTAR_EUNSUPPORTED;
    if (desc->R == 0) return NECTAR_OK;
    if (!tensor_ok(q) || !f32_ok(alpha_out) || !rows_ok(A_out)) return NECTAR_EINVAL;
    if (n > 0 && (!tensor_ok(k) || !tensor_ok(v))) return NECTAR_EINVAL;
    const AttnPlan pl = plan_doc(desc, (long)n);
    if ((s = check_ws(pl.ws, ws, ws_bytes)) != NECTAR_OK) return s;
    CombineParams cp{};
    cp.lse_out = alpha_out;
    cp.A_out = A_out;
    hipStream_t st = (hipStream_t)stream;
    return finish(run_attention(desc, pl, q, k, v, 0, (int64_t)n * doc_row(desc), doc_row(desc), 1, desc->R, (long)n, 0, 0,
                                cp, ws, st), st);
}

// ---------------------------------------------------------------------------
// Deep MLP module (Eq. (3.6) with re-injection): layer bookkeeping.

// Layer l's part (0 backbone, 1 score, 2 target), its width and the width of
// the state it reads (0: the query only).
struct DeepShape {
    int D[3], H[3], nl;
    int part(int l) const { return l < D[0] ? 0 : (l < D[0] + D[1] ? 1 : 2); }
    int first(int part) const { return part == 0 ? 0 : (part == 1 ? D[0] : D[0] + D[1]); }
    int in_width(int l) const {
        const int pt = part(l);
        return l > first(pt) ? H[pt] : (pt > 0 && D[0] > 0 ? H[0] : 0);
    }
    // width of the state a head's read-out reads
    int last_width(int head) const { return D[head] > 0 ? H[head] : H[0]; }
};

static DeepShape deep_shape(const nectar_deep_mlp *m) {
    DeepShape sh;
    for (int i = 0; i < 3; ++i) {
        sh.D[i] = m->depth[i];
        sh.H[i] = m->depth[i] > 0 ? m->width[i] : 0;
    }
    sh.nl = sh.D[0] + sh.D[1] + sh.D[2];
    return sh;
}

static nectar_status check_deep(const nectar_deep_mlp *m) {
    if (!m) return NECTAR_EINVAL;
    if (m->act != NECTAR_ACT_GELU && m->act != NECTAR_ACT_SILU && m->act != NECTAR_ACT_GELU_TANH)
        return NECTAR_EINVAL;
    for (int i = 0; i < 3; ++i)
        if (m->depth[i] < 0 || (m->depth[i] > 0 && m->width[i] <= 0)) return NECTAR_EINVAL;
    const DeepShape sh = deep_shape(m);
    if (sh.D[0] + sh.D[1] < 1 || sh.D[0] + sh.D[2] < 1) return NECTAR_EINVAL;
    if (sh.nl > NECTAR_DEEP_MAX_LAYERS) return NECTAR_EUNSUPPORTED;
    for (int i = 0; i < 3; ++i)
        if (sh.D[i] > 0 && (sh.H[i] % 32 != 0 || sh.H[i] > (1 << 20))) return NECTAR_EUNSUPPORTED;
    for (int l = 0; l < sh.nl; ++l) {
        if (!tensor_ok(m->Wq[l]) || !m->b[l] || !aligned(m->b[l], 4)) return NECTAR_EINVAL;
        if ((sh.in_width(l) > 0) != (m->Wh[l] != nullptr)) return NECTAR_EINVAL;
        if (m->Wh[l] && !tensor_ok(m->Wh[l])) return NECTAR_EINVAL;
    }
    if (!tensor_ok(m->ws_out) || !tensor_ok(m->Wt_out)) return NECTAR_EINVAL;
    if (!m->bs_out || !aligned(m->bs_out, 4) || !m->bt_out || !aligned(m->bt_out, 4)) return NECTAR_EINVAL;
    return NECTAR_OK;
}

// Rows per KV head from which a deep layer runs on the LDS-staged kernel.
#ifndef NECTAR_DEEP_LDS_ROWS
#define NECTAR_DEEP_LDS_ROWS 1024
#endif
static constexpr int kDeepLdsRows = NECTAR_DEEP_LDS_ROWS;

// Workspace: two ping-pong hidden-state buffers per part, [Hkv][Rp][H] each.
static size_t deep_buffer_bytes(const nectar_attn_desc *d, int H) {
    const size_t esz = d->dtype == NECTAR_BF16 ? 2 : 4;
    return align256((size_t)d->Hkv * d->R * (d->Hq / d->Hkv) * H * esz);
}

static size_t deep_ws_bytes(const nectar_attn_desc *d, const nectar_deep_mlp *m) {
    const DeepShape sh = deep_shape(m);
    size_t b = 0;
    for (int i = 0; i < 3; ++i) b += 2 * deep_buffer_bytes(d, sh.H[i]);
    return b;
}

static hipError_t run_deep(const nectar_attn_desc *desc, const nectar_deep_mlp *m, const void *q, float *a_out,
                           float *A_out, void *ws, hipStream_t st) {
    const DeepShape sh = deep_shape(m);
    const int G = desc->Hq / desc->Hkv, Rp = desc->R * G;
    char *buf[3][2];
    char *w = (char *)ws;
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 2; ++j) {
            buf[i][j] = w;
            w += deep_buffer_bytes(desc, sh.H[i]);
        }
    DeepParams a{};
    a.q = q; a.Hq = desc->Hq; a.G = G; a.Hkv = desc->Hkv; a.Rp = Rp;
    const int lds = desc->dtype == NECTAR_BF16 && Rp >= kDeepLdsRows;
    auto layer = [&](int l, int step) {
        const int pt = sh.part(l);
        DeepLayer L{};
        L.Wq = m->Wq[l]; L.Wh = m->Wh[l]; L.b = m->b[l];
        L.N = sh.H[pt]; L.Kh = sh.in_width(l); L.act = m->act;
        // the state read: the previous layer of the part, else the backbone's last
        if (l > sh.first(pt)) L.X = buf[pt][(step - 1) & 1];
        else if (L.Kh > 0) L.X = buf[0][(sh.D[0] - 1) & 1];
        L.Y = buf[pt][step & 1];
        L.blocks = deep_layer_blocks(desc->dtype, lds, desc->Hkv, Rp, L.N);
        return L;
    };
    auto head_state = [&](int head) -> const void * {
        return sh.D[head] > 0 ? buf[head][(sh.D[head] - 1) & 1] : buf[0][(sh.D[0] - 1) & 1];
    };
    hipError_t e = hipSuccess;
    for (int l = 0; l < sh.D[0] && e == hipSuccess; ++l) {
        a.nl = 1;
        a.L0 = layer(l, l);
        e = launch_deep_layers(a, desc->dtype, desc->d, lds, st);
    }
    const int Dh = sh.D[1] > sh.D[2] ? sh.D[1] : sh.D[2];
    for (int j = 0; j < Dh && e == hipSuccess; ++j) {
        a.nl = 0;
        if (j < sh.D[1]) a.L0 = layer(sh.first(1) + j, j), a.nl = 1;
        if (j < sh.D[2]) (a.nl ? a.L1 : a.L0) = layer(sh.first(2) + j, j), a.nl += 1;
        e = launch_deep_layers(a, desc->dtype, desc->d, lds, st);
    }
    if (e != hipSuccess) return e;
    // the two linear read-outs in one launch
    DeepLayer rs{}, rt{};
    rs.Wh = m->ws_out; rs.b = m->bs_out; rs.X = head_state(1); rs.Yf = a_out;
    rs.N = 1; rs.Kh = sh.last_width(1); rs.act = -1;
    rs.blocks = deep_layer_blocks(desc->dtype, lds, desc->Hkv, Rp, 1);
    rt.Wh = m->Wt_out; rt.b = m->bt_out; rt.X = head_state(2); rt.Yf = A_out;
    rt.N = desc->d; rt.Kh = sh.last_width(2); rt.act = -1;
    rt.blocks = deep_layer_blocks(desc->dtype, lds, desc->Hkv, Rp, desc->d);
    a.nl = 2; a.L0 = rs; a.L1 = rt;
    return launch_deep_layers(a, desc->dtype, desc->d, lds, st);
}

static nectar_status check_module(const nectar_attn_desc *desc, const nectar_module *m) {
    if (!m) return NECTAR_EINVAL;
    if (m->kind == NECTAR_MODULE_MLP) {
        if (m->act != NECTAR_ACT_GELU && m->act != NECTAR_ACT_SILU && m->act != NECTAR_ACT_GELU_TANH)
            return NECTAR_EINVAL;
        if (m->Ht < 0 || m->Hs < 0) return NECTAR_EINVAL;
        if (!m->b2 || !m->bs2 || !aligned(m->b2, 4) || !aligned(m->bs2, 4)) return NECTAR_EINVAL;
        if (m->Ht > 0 && (!tensor_ok(m->W1) || !tensor_ok(m->W2t) || !m->b1 || !aligned(m->b1, 4)))
            return NECTAR_EINVAL;
        if (m->Hs > 0 && (!tensor_ok(m->Ws) || !m->ws2 || !aligned(m->ws2, desc->dtype ? 2 : 4) ||
                          !m->bs || !aligned(m->bs, 4)))
            return NECTAR_EINVAL;
        return NECTAR_OK;
    }
    if (m->kind == NECTAR_MODULE_KVPAIR) {
        if (m->p < 0) return NECTAR_EINVAL;
        if (m->p > 0x7fffffffL - kTile) return NECTAR_EUNSUPPORTED;
        if (m->p > 0 && (!tensor_ok(m->W) || !tensor_ok(m->Z))) return NECTAR_EINVAL;
        return NECTAR_OK;
    }
    if (m->kind == NECTAR_MODULE_DEEP_MLP) return check_deep(m->deep);
    return NECTAR_EINVAL;
}

size_t nectar_module_workspace_size(const nectar_attn_desc *desc, const nectar_module *m) {
    if (check_desc(desc) != NECTAR_OK || !m) return 0;
    if (m->kind == NECTAR_MODULE_KVPAIR) {
        if (m->p < 0 || m->p > 0x7fffffffL - kTile) return 0;
        return plan_attn(desc, desc->Hkv, desc->R * (desc->Hq / desc->Hkv), (long)m->p).ws;
    }
    if (m->kind == NECTAR_MODULE_DEEP_MLP) return check_deep(m->deep) == NECTAR_OK ? deep_ws_bytes(desc, m->deep) : 0;
    if (m->kind != NECTAR_MODULE_MLP || m->Ht < 0 || m->Hs < 0) return 0;
    return plan_mlp(desc, m->Ht, m->Hs).ws;
}

// The MLP module forward of a plan: partial kernel, then the split reduce
// unless the partial kernel finished the rows itself.
static hipError_t run_mlp(const nectar_attn_desc *desc, const MlpPlan &pl, const nectar_module *m, const void *q,
                          float *a_out, float *A_out, void *ws, hipStream_t st) {
    float *part_O = (float *)ws;
    float *part_s = (float *)((char *)ws + (size_t)desc->Hkv * pl.SB * pl.Rp * desc->d * 4);
    MlpParams a{};
    a.q = q; a.W1 = m->W1; a.W2t = m->W2t; a.Ws = m->Ws; a.ws2 = m->ws2;
    a.b1 = m->b1; a.bs = m->bs; a.b2 = m->b2; a.bs2 = m->bs2;
    a.Hq = desc->Hq; a.G = desc->Hq / desc->Hkv; a.Hkv = desc->Hkv; a.Rp = pl.Rp;
    a.Ht = m->Ht; a.Hs = m->Hs; a.act = m->act;
    a.S = pl.S; a.chunk_t = pl.ct; a.chunk_s = pl.cs; a.RG = pl.RG;
    a.WR = pl.WR; a.WS = pl.WS; a.RB = pl.RB; a.SB = pl.SB; a.nwt = pl.Wt; a.nws = pl.Ws;
    a.part_O = part_O; a.part_s = part_s;
    a.a_out = a_out; a.A_out = A_out;
    const bool in_place = pl.SB == 1 && (pl.prefill || desc->dtype == NECTAR_BF16);
    hipError_t e = pl.dec ? launch_mlp_decode(a, desc->d, pl.RT, st)
                          : pl.lds32 ? launch_mlp_rows_lds32(a, st)
                                     : (pl.prefill ? launch_mlp_prefill(a, st)
                                                   : launch_mlp_partial(a, desc->dtype, desc->d, pl.RT, st));
    if (e == hipSuccess && !in_place) {
        MlpReduceParams r;
        r.part_O = part_O; r.part_s = part_s; r.b2 = m->b2; r.bs2 = m->bs2;
        r.Hq = desc->Hq; r.G = desc->Hq / desc->Hkv; r.Hkv = desc->Hkv; r.Rp = pl.Rp; r.S = pl.SB;
        r.a_out = a_out; r.A_out = A_out;
        e = launch_mlp_reduce(r, desc->d, st);
    }
    return e;
}

nectar_status nectar_module_forward(const nectar_attn_desc *desc, const nectar_module *m,
                                    const void *q, float *a_out, float *A_out, void *ws,
                                    size_t ws_bytes, void *stream) {
    nectar_status s = check_desc(desc);
    if (s != NECTAR_OK) return s;
    if ((s = check_module(desc, m)) != NECTAR_OK) return s;
    if (desc->R == 0) return NECTAR_OK;
    if (!tensor_ok(q) || !f32_ok(a_out) || !rows_ok(A_out)) return NECTAR_EINVAL;
    hipStream_t st = (hipStream_t)stream;
    if (m->kind == NECTAR_MODULE_KVPAIR) {
        const AttnPlan pl = plan_attn(desc, desc->Hkv, desc->R * (desc->Hq / desc->Hkv), (long)m->p);
        if ((s = check_ws(pl.ws, ws, ws_bytes)) != NECTAR_OK) return s;
        CombineParams cp{};
        cp.lse_out = a_out;
        cp.A_out = A_out;
        return finish(run_attention(desc, pl, q, m->W, m->Z, 0, m->p * desc->d, desc->d, 1, desc->R, (long)m->p,
                                    0, 0, cp, ws, st), st);
    }
    if (m->kind == NECTAR_MODULE_DEEP_MLP) {
        if ((s = check_ws(deep_ws_bytes(desc, m->deep), ws, ws_bytes)) != NECTAR_OK) return s;
        return finish(run_deep(desc, m->deep, q, a_out, A_out, ws, st), st);
    }
    const MlpPlan pl = plan_mlp(desc, m->Ht, m->Hs);
    if ((s = check_ws(pl.ws, ws, ws_bytes)) != NECTAR_OK) return s;
    return finish(run_mlp(desc, pl, m, q, a_out, A_out, ws, st), st);
}

static nectar_status check_local(const nectar_attn_desc *desc, const nectar_local_desc *loc) {
    if (!loc) return NECTAR_EINVAL;
    if (loc->B < 0 || loc->Tq < 0 || (long)loc->B * loc->Tq != desc->R) return NECTAR_EINVAL;
    if (loc->T_loc < 0 || loc->T_cap < loc->T_loc || loc->q_offset < 0) return NECTAR_EINVAL;
    if (loc->T_loc > 0x7fffffff - kTile) return NECTAR_EUNSUPPORTED;
    return NECTAR_OK;
}

size_t nectar_local_workspace_size(const nectar_attn_desc *desc, const nectar_local_desc *loc) {
    if (check_desc(desc) != NECTAR_OK || check_local(desc, loc) != NECTAR_OK) return 0;
    return plan_attn(desc, loc->B * desc->Hkv, loc->Tq * (desc->Hq / desc->Hkv), loc->T_loc).ws;
}

nectar_status nectar_local_attn_lse(const nectar_attn_desc *desc, const nectar_local_desc *loc,
                                    const void *q, const void *k_loc, const void *v_loc,
                                    float *lse_out, float *A_out, const float *doc_lse,
                                    const float *doc_A, void *out, float *out_lse, void *ws,
                                    size_t ws_bytes, void *stream) {
    nectar_status s = check_desc(desc);
    if (s != NECTAR_OK) return s;
    if ((s = check_local(desc, loc)) != NECTAR_OK) return s;
    const bool want_merge = out || out_lse;
    if (!lse_out && !A_out && !want_merge) return NECTAR_EINVAL;
    if (want_merge != (doc_lse || doc_A)) return NECTAR_EINVAL;
    if (want_merge && (!f32_ok(doc_lse) || !rows_ok(doc_A))) return NECTAR_EINVAL;
    if ((lse_out && !f32_ok(lse_out)) || (A_out && !rows_ok(A_out)) || (out && !rows_ok(out)) ||
        (out_lse && !f32_ok(out_lse)))
        return NECTAR_EINVAL;
    if (desc->R == 0) return NECTAR_OK;
    if (!tensor_ok(q)) return NECTAR_EINVAL;
    if (loc->T_loc > 0 && (!tensor_ok(k_loc) || !tensor_ok(v_loc))) return NECTAR_EINVAL;
    const AttnPlan pl = plan_attn(desc, loc->B * desc->Hkv, loc->Tq * (desc->Hq / desc->Hkv), loc->T_loc);
    if ((s = check_ws(pl.ws, ws, ws_bytes)) != NECTAR_OK) return s;
    CombineParams cp{};
    cp.lse_out = lse_out;
    cp.A_out = A_out;
    cp.x_lse = doc_lse;
    cp.x_A = doc_A;
    cp.out = out;
    cp.out_lse = out_lse;
    hipStream_t st = (hipStream_t)stream;
    const int64_t hstride = (int64_t)loc->T_cap * desc->d;
    return finish(run_attention(desc, pl, q, k_loc, v_loc, hstride * desc->Hkv, hstride, desc->d, loc->B, loc->Tq,
                                loc->T_loc, 1, loc->q_offset, cp, ws, st), st);
}

nectar_status nectar_merge(const nectar_attn_desc *desc, const float *a, const float *A, const float *lam,
                           const float *A_loc, void *out, float *lse_out, void *stream) {
    nectar_status s = check_desc(desc);
    if (s != NECTAR_OK) return s;
    if (desc->R == 0) return NECTAR_OK;
    if (!f32_ok(a) || !rows_ok(A) || !f32_ok(lam) || !rows_ok(A_loc) || !rows_ok(out))
        return NECTAR_EINVAL;
    if (lse_out && !f32_ok(lse_out)) return NECTAR_EINVAL;
    MergeParams p;
    p.a = a; p.A = A; p.lam = lam; p.A_loc = A_loc; p.out = out; p.lse_out = lse_out;
    p.rows = (long)desc->R * desc->Hq;
    hipStream_t st = (hipStream_t)stream;
    return finish(launch_merge(p, desc->dtype, desc->d, st), st);
}

nectar_status nectar_merge_k(const nectar_attn_desc *desc, int K, const float *const *a,
                             const float *const *A, const float *lam, const float *A_loc, void *out,
                             float *lse_out, void *stream) {
    nectar_status s = check_desc(desc);
    if (s != NECTAR_OK) return s;
    if (K < 0 || K > NECTAR_MERGE_K_MAX) return NECTAR_EINVAL;
    if ((lam == nullptr) != (A_loc == nullptr)) return NECTAR_EINVAL;
    if (K == 0 && lam == nullptr) return NECTAR_EINVAL;
    if (K > 0 && (a == nullptr || A == nullptr)) return NECTAR_EINVAL;
    if (desc->R == 0) return NECTAR_OK;
    MergeKParams p = {};
    for (int k = 0; k < K; ++k) {
        if (!f32_ok(a[k]) || !rows_ok(A[k])) return NECTAR_EINVAL;
        p.a[k] = a[k];
        p.A[k] = A[k];
    }
    if (lam && (!f32_ok(lam) || !rows_ok(A_loc))) return NECTAR_EINVAL;
    if (!rows_ok(out)) return NECTAR_EINVAL;
    if (lse_out && !f32_ok(lse_out)) return NECTAR_EINVAL;
    p.lam = lam; p.A_loc = A_loc; p.out = out; p.lse_out = lse_out;
    p.rows = (long)desc->R * desc->Hq;
    p.K = K;
    hipStream_t st = (hipStream_t)stream;
    return finish(launch_merge_k(p, desc->dtype, desc->d, st), st);
}

size_t nectar_fit_metrics_workspace_size(const nectar_attn_desc *desc) {
    if (check_desc(desc) != NECTAR_OK) return 0;
    return (size_t)desc->Hkv * kFitParts * 3 * sizeof(double);
}

nectar_status nectar_fit_metrics(const nectar_attn_desc *desc, const void *q, const float *a, const float *A,
                                 const float *alpha, const float *A_exact, float *row_out, double *head_out,
                                 void *ws, size_t ws_bytes, void *stream) {
    nectar_status s = check_desc(desc);
    if (s != NECTAR_OK) return s;
    if (desc->R == 0) return NECTAR_OK;
    if (!tensor_ok(q) || !f32_ok(a) || !f32_ok(alpha) || !rows_ok(A) || !rows_ok(A_exact) || !f32_ok(row_out))
        return NECTAR_EINVAL;
    if (head_out) {
        if (!aligned(head_out, 8)) return NECTAR_EINVAL;
        if ((s = check_ws(nectar_fit_metrics_workspace_size(desc), ws, ws_bytes)) != NECTAR_OK) return s;
    }
    FitParams p{};
    p.q = q; p.a = a; p.A = A; p.alpha = alpha; p.Aex = A_exact;
    p.row = row_out; p.head = head_out; p.part = (double *)ws;
    p.rows = (long)desc->R * desc->Hq;
    p.Hq = desc->Hq; p.Hkv = desc->Hkv;
    hipStream_t st = (hipStream_t)stream;
    return finish(launch_fit_metrics(p, desc->dtype, desc->d, st), st);
}

// ---------------------------------------------------------------------------
// Regression training step of the one-hidden-layer module.

namespace {

constexpr int kTrainParts = 64, kMaxSplit = 8;

struct TrainLayout {
    int Rp = 0, Ht = 0, Hs = 0, d = 0, Hkv = 0;
    // fused (d = 128): the module's forward kernels, then one backward launch
    // that recomputes the pre-activations (rows padded to Rpad per group);
    // otherwise stored pre-activations and hidden values between products
    bool fused = false;
    int Rpad = 0;
    MlpPlan fwd;
    // flat parameter offsets (elements): W1, b1, W2t, b2, Ws, bs, ws2, bs2, total
    long off[9] = {};
    // workspace offsets (bytes)
    size_t Q, Zb, Yt, W2tT, Aout, gA, Zs, Ys, dZs, ga, es, et, Cpart, xsp, csp, parts, scale, bytes;
    size_t am, Am, fws;      // fused: the forward's (a, A) and its workspace
};

TrainLayout train_layout(const nectar_attn_desc *d, const nectar_module *m) {
    TrainLayout L;
    const long H = d->Hkv;
    L.Hkv = d->Hkv; L.d = d->d; L.Ht = m->Ht; L.Hs = m->Hs;
    L.Rp = d->R * (d->Hq / d->Hkv);
    const long sizes[8] = {H * L.Ht * L.d, H * L.Ht, H * L.Ht * L.d, H * L.d,
                           H * L.Hs * L.d, H * L.Hs, H * L.Hs, H};
    L.off[0] = 0;
    for (int i = 0; i < 8; ++i) L.off[i + 1] = L.off[i] + sizes[i];
    size_t o = 0;
    auto take = [&](size_t bytes) { const size_t at = o; o += align256(bytes); return at; };
    L.fused = d->d == 128 && d->dtype == NECTAR_BF16;
    if (L.fused) {
        L.Rpad = (int)cdiv(L.Rp, 64) * 64;      // whole 64-row stages of the backward
        L.fwd = plan_mlp(d, L.Ht, L.Hs);
        const size_t Rq = (size_t)d->R * d->Hq, Rr = (size_t)H * L.Rp, Rd = (size_t)H * L.Rpad;
        L.Q = take(Rd * L.d * 2);
        L.gA = take(Rd * L.d * 2);
        L.ga = take(Rd * 4);
        L.es = take(Rr * 4);
        L.et = take(Rr * 4);
        L.am = take(Rq * 4);
        L.Am = take(Rq * L.d * 4);
        L.fws = take(L.fwd.ws);
        L.csp = take((size_t)H * ((L.Rp + 63) / 64) * L.d * 4);
        L.parts = take((2 * kTrainParts + kNormParts) * 8);
        L.scale = take(2 * 4);
        L.bytes = o;
        return L;
    }
    const size_t R = (size_t)H * L.Rp;
    L.Q = take(R * L.d * 2);
    L.Zb = take(R * L.Ht * 2);
    L.Yt = take(R * L.Ht * 2);
    L.W2tT = take((size_t)H * L.d * L.Ht * 2);
    L.Aout = take(R * L.d * 4);
    L.gA = take(R * L.d * 2);
    L.Zs = take(R * L.Hs * 4);
    L.Ys = take(R * L.Hs * 2);
    L.dZs = take(R * L.Hs * 2);
    L.ga = take(R * 4);
    L.es = take(R * 4);
    L.et = take(R * 4);
    L.Cpart = take((size_t)kMaxSplit * H * std::max(std::max(L.Rp, L.Ht), L.Hs) * L.d * 4);
    L.xsp = take((size_t)kMaxSplit * H * std::max(L.Ht, L.Hs) * 4);
    L.csp = take((size_t)H * ((L.Rp + 63) / 64) * std::max(L.Hs, L.d) * 4);
    L.parts = take((2 * kTrainParts + kNormParts) * 8);
    L.scale = take(2 * 4);
    L.bytes = o;
    return L;
}

nectar_status check_train(const nectar_attn_desc *desc, const nectar_module *m) {
    nectar_status s = check_desc(desc);
    if (s != NECTAR_OK) return s;
    if ((s = check_module(desc, m)) != NECTAR_OK) return s;
    if (m->kind != NECTAR_MODULE_MLP) return NECTAR_EUNSUPPORTED;
    if (desc->dtype != NECTAR_BF16) return NECTAR_EUNSUPPORTED;
    if (m->Ht <= 0 || m->Hs <= 0 || m->Ht % 32 || m->Hs % 32) return NECTAR_EUNSUPPORTED;
    if (desc->R <= 0) return NECTAR_EINVAL;
    return NECTAR_OK;
}

GemmParams gemm(const void *X, long sx, int ldx, const void *W, long sw, int ldw, const float *bias, long sb,
                float *C, long sc, int ldc, int M, int N, int K, int P) {
    GemmParams g{};
    g.X = (const uint16_t *)X; g.W = (const uint16_t *)W; g.bias = bias; g.C = C;
    g.sx = sx; g.sw = sw; g.sb = sb; g.sc = sc; g.ldx = ldx; g.ldw = ldw; g.ldc = ldc;
    g.M = M; g.N = N; g.K = K; g.P = P;
    g.ksplit = 1; g.kchunk = K;
    return g;
}

// Split the contraction of a product whose tiles alone would leave most CUs
// idle (partial tiles in Cpart, then a fixed-order reduce).
GemmParams with_split(GemmParams g, float *Cpart) {
    const long b = gemm_blocks(g);
    if (b >= 512 || g.K < 1024 || g.N % 4) return g;
    int ks = (int)std::min<long>(kMaxSplit, (512 + b - 1) / b);
    const int kc = ((g.K + ks - 1) / ks + 31) / 32 * 32;
    ks = (g.K + kc - 1) / kc;
    if (ks > 1) {
        g.ksplit = ks;
        g.kchunk = kc;
        g.Cpart = Cpart;
    }
    return g;
}

TransposeParams transpose(const void *in, long si, int ldi, void *out, long so, int ldo, int rows, int cols, int P) {
    TransposeParams t{};
    t.in = (const uint16_t *)in; t.out = (uint16_t *)out; t.si = si; t.so = so;
    t.rows = rows; t.cols = cols; t.ldi = ldi; t.ldo = ldo; t.P = P;
    return t;
}

RowDotParams rowdot(const void *X, long sx, int ldx, const float *v, long sv, float *out, long so, int J, int K, int P) {
    RowDotParams r{};
    r.X = X; r.sx = sx; r.ldx = ldx; r.v = v; r.sv = sv; r.out = out; r.so = so; r.J = J; r.K = K; r.P = P;
    return r;
}

// Fused loss and gradient (d = 128): (a, A) from the module's forward kernels,
// the residual rows, one backward launch for every weight, hidden-bias and
// score read-out gradient, then the output-bias gradients as fixed-order sums.
hipError_t run_loss_grad_fused(const nectar_attn_desc *desc, const nectar_module *m, const TrainLayout &L,
                               const void *q, const float *alpha, const float *Atgt, float lam_alpha, float lam_A,
                               float *grad, char *w, hipStream_t st) {
    const int P = L.Hkv, Rp = L.Rp, Rpad = L.Rpad, d = L.d;
    auto F = [&](size_t off) { return (float *)(w + off); };
    hipError_t e = hipSuccess;
    auto run = [&](hipError_t x) { if (e == hipSuccess) e = x; };
    GatherParams gq{};
    gq.q = (const uint16_t *)q; gq.Q = (uint16_t *)(w + L.Q);
    gq.Hq = desc->Hq; gq.G = desc->Hq / desc->Hkv; gq.Hkv = P; gq.Rp = Rp; gq.d = d; gq.Rpad = Rpad;
    run(launch_gather_q(gq, st));
    if (e == hipSuccess) e = run_mlp(desc, L.fwd, m, q, F(L.am), F(L.Am), w + L.fws, st);
    LossRowParams lr{};
    lr.a = F(L.am); lr.A = F(L.Am); lr.alpha = alpha; lr.Atgt = Atgt;
    lr.gA = (uint16_t *)(w + L.gA); lr.ga = F(L.ga); lr.es = F(L.es); lr.et = F(L.et);
    lr.coefa = 2.0f * lam_alpha / (float)desc->R;
    lr.coefA = 2.0f * lam_A / (float)desc->R;
    lr.Hq = desc->Hq; lr.G = desc->Hq / desc->Hkv; lr.Hkv = P; lr.Rp = Rp; lr.Rpad = Rpad;
    run(launch_loss_rows(lr, st));
    TrainBwdParams tb{};
    tb.Q = (const uint16_t *)(w + L.Q); tb.gA = (const uint16_t *)(w + L.gA); tb.ga = F(L.ga);
    tb.W1 = (const uint16_t *)m->W1; tb.W2t = (const uint16_t *)m->W2t; tb.Ws = (const uint16_t *)m->Ws;
    tb.ws2 = (const uint16_t *)m->ws2; tb.b1 = m->b1; tb.bs = m->bs;
    tb.gW1 = grad + L.off[0]; tb.gb1 = grad + L.off[1]; tb.gW2t = grad + L.off[2];
    tb.gWs = grad + L.off[4]; tb.gbs = grad + L.off[5]; tb.gws2 = grad + L.off[6]; tb.gbs2 = grad + L.off[7];
    tb.Hkv = P; tb.Rpad = Rpad; tb.Ht = L.Ht; tb.Hs = L.Hs;
    tb.nut = (int)cdiv(L.Ht, 128); tb.nus = (int)cdiv(L.Hs, 128); tb.items = P * (tb.nut + tb.nus);
    run(launch_train_bwd(tb, m->act, st));
    // db2 = column sums of gA (dbs2, the sums of ga, come from the backward)
    ColSumParams c{};
    c.X = (const uint16_t *)(w + L.gA); c.v = nullptr; c.parts = F(L.csp); c.out = grad + L.off[3];
    c.sx = (long)Rpad * d; c.sv = Rpad; c.so = d; c.ldx = d; c.rows = Rp; c.cols = d; c.P = P;
    run(launch_col_sum(c, st));
    SumParams su{};
    su.parts = (double *)(w + L.parts);
    su.x = F(L.es); su.n = (long)P * Rp; su.part0 = 0; su.square = 0;
    run(launch_sum_parts(su, kTrainParts, st));
    su.x = F(L.et); su.part0 = kTrainParts;
    run(launch_sum_parts(su, kTrainParts, st));
    return e;
}

// Loss terms and gradient into grad (flat fp32, parameter order of TrainLayout).
hipError_t run_loss_grad(const nectar_attn_desc *desc, const nectar_module *m, const TrainLayout &L, const void *q,
                         const float *alpha, const float *Atgt, float lam_alpha, float lam_A, float *grad,
                         char *w, hipStream_t st) {
    const int P = L.Hkv, Rp = L.Rp, d = L.d, Ht = L.Ht, Hs = L.Hs;
    auto B = [&](size_t off) { return (void *)(w + off); };
    auto F = [&](size_t off) { return (float *)(w + off); };
    hipError_t e = hipSuccess;
    auto run = [&](hipError_t x) { if (e == hipSuccess) e = x; };
    if (L.fused) return run_loss_grad_fused(desc, m, L, q, alpha, Atgt, lam_alpha, lam_A, grad, w, st);

    GatherParams gq{};
    gq.q = (const uint16_t *)q; gq.Q = (uint16_t *)B(L.Q);
    gq.Hq = desc->Hq; gq.G = desc->Hq / desc->Hkv; gq.Hkv = P; gq.Rp = Rp; gq.d = d;
    run(launch_gather_q(gq, st));
    // forward: pre-activations (bias included), hidden values, read-out
    GemmParams gz = gemm(B(L.Q), (long)Rp * d, d, m->W1, (long)Ht * d, d, m->b1, Ht, nullptr, (long)Rp * Ht, Ht,
                         Rp, Ht, d, P);
    gz.epi = 1; gz.act = m->act; gz.Zo = (uint16_t *)B(L.Zb); gz.Y = (uint16_t *)B(L.Yt);   // Z and act(Z), bf16
    run(launch_gemm_nt(gz, st));
    run(launch_gemm_nt(gemm(B(L.Q), (long)Rp * d, d, m->Ws, (long)Hs * d, d, m->bs, Hs, F(L.Zs), (long)Rp * Hs, Hs,
                            Rp, Hs, d, P), st));
    run(launch_transpose_bf16(transpose(m->W2t, (long)Ht * d, d, B(L.W2tT), (long)d * Ht, Ht, Ht, d, P), st));
    run(launch_gemm_nt(with_split(gemm(B(L.Yt), (long)Rp * Ht, Ht, B(L.W2tT), (long)d * Ht, Ht, m->b2, d,
                                       F(L.Aout), (long)Rp * d, d, Rp, d, Ht, P), F(L.Cpart)), st));
    // loss terms and the output gradients
    TargetRowParams tp{};
    tp.A = F(L.Aout); tp.Atgt = Atgt; tp.gA = (uint16_t *)B(L.gA); tp.err = F(L.et);
    tp.coef = 2.0f * lam_A / (float)desc->R;
    tp.Hq = desc->Hq; tp.G = desc->Hq / desc->Hkv; tp.Hkv = P; tp.Rp = Rp;
    run(launch_target_rows(tp, d, st));
    ScoreRowParams sp{};
    sp.Zs = F(L.Zs); sp.ws2 = (const uint16_t *)m->ws2; sp.bs2 = m->bs2; sp.alpha = alpha;
    sp.Ys = (uint16_t *)B(L.Ys); sp.dZs = (uint16_t *)B(L.dZs); sp.ga = F(L.ga); sp.err = F(L.es);
    sp.coef = 2.0f * lam_alpha / (float)desc->R;
    sp.Hq = desc->Hq; sp.G = desc->Hq / desc->Hkv; sp.Hkv = P; sp.Rp = Rp; sp.Hs = Hs;
    run(launch_score_rows(sp, m->act, st));
    // weight gradients: contractions over the rows of the row-major buffers
    // (TN products), bias gradients as fixed-order column sums
    float *gW1 = grad + L.off[0], *gb1 = grad + L.off[1], *gW2t = grad + L.off[2], *gb2 = grad + L.off[3];
    float *gWs = grad + L.off[4], *gbs = grad + L.off[5], *gws2 = grad + L.off[6], *gbs2 = grad + L.off[7];
    auto colsum = [&](const void *X, long sx, int ldx, int cols, const float *v, float *out, long so) {
        ColSumParams c{};
        c.X = (const uint16_t *)X; c.v = v; c.parts = F(L.csp); c.out = out;
        c.sx = sx; c.sv = Rp; c.so = so; c.ldx = ldx; c.rows = Rp; c.cols = cols; c.P = P;
        run(launch_col_sum(c, st));
    };
    // target read-out: dW2t = Y^T gA (before Y's buffer takes dZ_t), db2 = column sums of gA
    run(launch_gemm_tn(with_split(gemm(B(L.Yt), (long)Rp * Ht, Ht, B(L.gA), (long)Rp * d, d, nullptr, 0, gW2t,
                                       (long)Ht * d, d, Ht, d, Rp, P), F(L.Cpart)), st));
    colsum(B(L.gA), (long)Rp * d, d, d, nullptr, gb2, d);
    // dZ_t = (gA W2t) * act'(Z), bf16, into the hidden-value buffer (no longer needed)
    GemmParams gd = gemm(B(L.gA), (long)Rp * d, d, m->W2t, (long)Ht * d, d, nullptr, 0, nullptr, (long)Rp * Ht, Ht,
                         Rp, Ht, d, P);
    gd.epi = 2; gd.act = m->act; gd.Zi = (const uint16_t *)B(L.Zb); gd.Y = (uint16_t *)B(L.Yt);
    run(launch_gemm_nt(gd, st));
    // first layers: dW1 = dZ_t^T Q, dWs = dZ_s^T Q; their biases; the score read-out
    // (the bias gradients db1, dbs are the column sums of the X operands, formed
    // inside the same products)
    auto with_xsum = [&](GemmParams g, float *xsum, long sxs) {
        g.xsum = xsum; g.xsum_part = F(L.xsp); g.sxs = sxs;
        return g;
    };
    run(launch_gemm_tn(with_xsum(with_split(gemm(B(L.Yt), (long)Rp * Ht, Ht, B(L.Q), (long)Rp * d, d, nullptr, 0,
                                                 gW1, (long)Ht * d, d, Ht, d, Rp, P), F(L.Cpart)), gb1, Ht), st));
    run(launch_gemm_tn(with_xsum(with_split(gemm(B(L.dZs), (long)Rp * Hs, Hs, B(L.Q), (long)Rp * d, d, nullptr, 0,
                                                 gWs, (long)Hs * d, d, Hs, d, Rp, P), F(L.Cpart)), gbs, Hs), st));
    colsum(B(L.Ys), (long)Rp * Hs, Hs, Hs, F(L.ga), gws2, Hs);
    run(launch_row_dot(rowdot(F(L.ga), Rp, Rp, nullptr, 0, gbs2, 1, 1, Rp, P), 1, st));
    // loss sums
    SumParams su{};
    su.parts = (double *)B(L.parts);
    su.x = F(L.es); su.n = (long)P * Rp; su.part0 = 0; su.square = 0;
    run(launch_sum_parts(su, kTrainParts, st));
    su.x = F(L.et); su.part0 = kTrainParts;
    run(launch_sum_parts(su, kTrainParts, st));
    return e;
}

}  // namespace

int64_t nectar_mlp_param_count(const nectar_attn_desc *desc, const nectar_module *m) {
    if (check_desc(desc) != NECTAR_OK || !m || m->kind != NECTAR_MODULE_MLP || m->Ht < 0 || m->Hs < 0) return 0;
    const long H = desc->Hkv, d = desc->d;
    return H * (2L * m->Ht * d + m->Ht + d + m->Hs * d + 2L * m->Hs + 1);
}

size_t nectar_mlp_train_workspace_size(const nectar_attn_desc *desc, const nectar_module *m) {
    if (check_train(desc, m) != NECTAR_OK) return 0;
    return train_layout(desc, m).bytes;
}

nectar_status nectar_mlp_loss_grad(const nectar_attn_desc *desc, const nectar_module *m, const void *q,
                                   const float *alpha, const float *A_target, float lambda_alpha, float lambda_A,
                                   float *grad, float *loss, void *ws, size_t ws_bytes, void *stream) {
    nectar_status s = check_train(desc, m);
    if (s != NECTAR_OK) return s;
    if (!tensor_ok(q) || !f32_ok(alpha) || !rows_ok(A_target) || !rows_ok(grad) || !f32_ok(loss))
        return NECTAR_EINVAL;
    if (!std::isfinite(lambda_alpha) || !std::isfinite(lambda_A)) return NECTAR_EINVAL;
    const TrainLayout L = train_layout(desc, m);
    if ((s = check_ws(L.bytes, ws, ws_bytes)) != NECTAR_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    char *w = (char *)ws;
    hipError_t e = run_loss_grad(desc, m, L, q, alpha, A_target, lambda_alpha, lambda_A, grad, w, st);
    if (e == hipSuccess) {
        TrainScalars ts{};
        ts.parts = (const double *)(w + L.parts); ts.nparts = kTrainParts;
        ts.R = desc->R; ts.lam_alpha = lambda_alpha; ts.lam_A = lambda_A; ts.loss = loss;
        e = launch_train_scalars(ts, st);
    }
    return finish(e, st);
}

static bool hparams_ok(const nectar_train_hparams *hp) {
    return hp && hp->step >= 1 && std::isfinite(hp->lr) && hp->beta1 >= 0.f && hp->beta1 < 1.f && hp->beta2 >= 0.f &&
           hp->beta2 < 1.f && hp->eps > 0.f && std::isfinite(hp->weight_decay) && std::isfinite(hp->clip_norm) &&
           std::isfinite(hp->lambda_alpha) && std::isfinite(hp->lambda_A);
}

static AdamParams adam_params(const nectar_train_hparams *hp, float *theta, const float *g, float *m, float *v,
                              long n, const float *scale) {
    AdamParams a{};
    a.theta = theta; a.g = g; a.m = m; a.v = v; a.n = n; a.scale = scale;
    a.lr = hp->lr; a.b1 = hp->beta1; a.b2 = hp->beta2; a.eps = hp->eps; a.wd = hp->weight_decay;
    a.ic1 = (float)(1.0 / (1.0 - std::pow((double)hp->beta1, hp->step)));
    a.ic2 = (float)(1.0 / (1.0 - std::pow((double)hp->beta2, hp->step)));
    return a;
}

nectar_status nectar_adamw_step(int64_t n, float *theta, const float *grad, float *adam_m, float *adam_v,
                                const nectar_train_hparams *hp, void *stream) {
    if (n < 0 || !hparams_ok(hp)) return NECTAR_EINVAL;
    if (n == 0) return NECTAR_OK;
    if (!f32_ok(theta) || !f32_ok(grad) || !f32_ok(adam_m) || !f32_ok(adam_v)) return NECTAR_EINVAL;
    hipStream_t st = (hipStream_t)stream;
    return finish(launch_adamw(adam_params(hp, theta, grad, adam_m, adam_v, (long)n, nullptr), st), st);
}

nectar_status nectar_mlp_train_step(const nectar_attn_desc *desc, const nectar_module *m, const void *q,
                                    const float *alpha, const float *A_target, const nectar_train_hparams *hp,
                                    float *theta, float *adam_m, float *adam_v, float *grad, float *loss,
                                    float *gnorm, void *ws, size_t ws_bytes, void *stream) {
    nectar_status s = check_train(desc, m);
    if (s != NECTAR_OK) return s;
    if (!hparams_ok(hp)) return NECTAR_EINVAL;
    if (!tensor_ok(q) || !f32_ok(alpha) || !rows_ok(A_target) || !rows_ok(grad) || !rows_ok(theta) ||
        !rows_ok(adam_m) || !rows_ok(adam_v))
        return NECTAR_EINVAL;
    if ((loss && !f32_ok(loss)) || (gnorm && !f32_ok(gnorm))) return NECTAR_EINVAL;
    const TrainLayout L = train_layout(desc, m);
    if ((s = check_ws(L.bytes, ws, ws_bytes)) != NECTAR_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    char *w = (char *)ws;
    hipError_t e = run_loss_grad(desc, m, L, q, alpha, A_target, hp->lambda_alpha, hp->lambda_A, grad, w, st);
    const long n = L.off[8];
    if (e == hipSuccess) {
        SumParams su{};
        su.parts = (double *)(w + L.parts); su.x = grad; su.n = n; su.part0 = 2 * kTrainParts; su.square = 1;
        e = launch_sum_parts(su, kNormParts, st);
    }
    float *scale = (float *)(w + L.scale);
    if (e == hipSuccess) {
        TrainScalars ts{};
        ts.parts = (const double *)(w + L.parts); ts.nparts = kTrainParts;
        ts.R = desc->R; ts.lam_alpha = hp->lambda_alpha; ts.lam_A = hp->lambda_A; ts.clip = hp->clip_norm;
        ts.loss = loss; ts.scale = scale; ts.gnorm = gnorm;
        e = launch_train_scalars(ts, st);
    }
    // AdamW, writing the module's arrays from the updated master parameters in
    // the same pass (weights rounded to bf16, biases copied)
    AdamParams ap = adam_params(hp, theta, grad, adam_m, adam_v, n, scale);
    const void *dst[8] = {m->W1, m->b1, m->W2t, m->b2, m->Ws, m->bs, m->ws2, m->bs2};
    ap.nseg = 8;
    ap.bf16 = (1 << 0) | (1 << 2) | (1 << 4) | (1 << 6);
    for (int i = 0; i < 9; ++i) ap.off[i] = L.off[i];
    for (int i = 0; i < 8; ++i) ap.dst[i] = const_cast<void *>(dst[i]);
    if (e == hipSuccess) e = launch_adamw(ap, st);
    return finish(e, st);
}

// ---------------------------------------------------------------------------
// Whole layer step: deferred partials of every part, one finishing pass.

// Partial bytes of an attention plan when its finish is deferred.
static size_t attn_partial_bytes(const nectar_attn_desc *d, const AttnPlan &pl) {
    return pl.S > 0 ? (size_t)pl.P * pl.SB * pl.Rp * ((size_t)d->d * 4 + 8) : 0;
}

static size_t mlp_partial_bytes(const nectar_attn_desc *d, const MlpPlan &pl) {
    return (size_t)d->Hkv * pl.SB * pl.Rp * ((size_t)d->d * 4 + 4);
}

struct StepPlan {
    bool exact = false, mlp = false, kvp = false, deep = false;
    size_t deep_ws = 0;
    // fused: deferred partials of every part, then one finishing launch (decode
    // shapes, where every part is short); otherwise the parts finish in place
    // or with their own combine and the local pass merges.
    bool fused = false;
    AttnPlan loc, doc, kvpl;
    MlpPlan mlpl;
    // Quadrature pairs (LDS-staged) and a decode local part in one launch: the
    // local part as LDS-staged blocks of the same shape beside the pairs'
    bool kvp_pair = false;
    size_t off_doc = 0, off_mod = 0;               // fused: partial regions
    size_t off_px = 0, off_pm = 0, off_pl = 0;     // composed: scratch pairs
    size_t off_po = 0;                             // composed: scratch merged output
    size_t bytes = 0;
};

static size_t pair_bytes(const nectar_attn_desc *d) {
    return align256((size_t)d->R * d->Hq * 4) + align256((size_t)d->R * d->Hq * d->d * 4);
}

static StepPlan plan_step(const nectar_attn_desc *d, int64_t n, const nectar_local_desc *loc,
                          const nectar_module *m, bool exact) {
    StepPlan sp;
    const int G = d->Hq / d->Hkv, Rp_doc = d->R * G;
    sp.loc = plan_attn(d, loc->B * d->Hkv, loc->Tq * G, loc->T_loc);
    sp.exact = exact;
    if (exact) sp.doc = plan_attn(d, d->Hkv, Rp_doc, (long)n);
    if (m && m->kind == NECTAR_MODULE_MLP) {
        sp.mlp = true;
        sp.mlpl = plan_mlp(d, m->Ht, m->Hs);
    } else if (m && m->kind == NECTAR_MODULE_DEEP_MLP) {
        sp.deep = true;
        sp.deep_ws = deep_ws_bytes(d, m->deep);
    } else if (m) {
        sp.kvp = true;
        sp.kvpl = plan_attn(d, d->Hkv, Rp_doc, (long)m->p);
    }
    auto decode = [](const AttnPlan &pl) { return pl.S == 0 || (!pl.lds && pl.RT == 1); };
    // A document-side attention may also be LDS-staged (many rows per KV head
    // beside a decode-shaped local part): its deferred partials go to the one
    // finishing pass, which saves its own combine launch and the merge.
    auto doc_side = [&](const AttnPlan &pl) { return decode(pl) || pl.lds; };
    // (with the document in the same launch the module has at most 16 rows per
    // KV head too, so both run one row tile)
    // A batched module (the LDS-staged kernels, 65+ rows per KV head) finishes
    // with its own split fold: its many split partials per row make the finishing
    // pass slower than that fold plus a merge (batch-64 decode layer, Nectar path:
    // 63.5 us composed, 72 us fused).
    sp.fused = !sp.deep && (d->dtype == NECTAR_F32 ||
               (decode(sp.loc) && (!exact || doc_side(sp.doc)) && (!sp.mlp || !sp.mlpl.prefill) &&
                (!sp.kvp || doc_side(sp.kvpl))));
    if (sp.fused) {
        if (sp.mlp && exact && !sp.doc.lds) sp.mlpl = plan_mlp(d, m->Ht, m->Hs, kTargetWavesMlpShared, true);
        // with a module in the same launch the document leaves 48 of the 512
        // two-per-CU block slots free from the start, so the module's blocks run
        // beside the document's instead of after them (4B step, waves left free
        // 96 / 128 / 160 / 192 / 256 / 352: 56.8 / 56.0 / 55.0 / 54.8 / 55.5 /
        // 56.9 us; all 512 slots to the document was 61.2 us with the earlier
        // finishing pass)
        if (exact && m && !sp.doc.lds) sp.doc = plan_attn(d, d->Hkv, Rp_doc, (long)n, true, kTargetWaves - 192);
        // exact path alone: the document leaves the local part's blocks their
        // slots, so both fill the 512 two-per-CU slots in one wave of blocks
        // (4B exact path 49.4 -> 48.5 us)
        else if (exact && d->dtype == NECTAR_BF16 && sp.loc.S > 0 && !sp.loc.lds && sp.loc.RT == 1) {
            const long loc_waves = 4L * sp.loc.P * sp.loc.RB * sp.loc.SB;
            if (loc_waves < kTargetWaves / 4) sp.doc = plan_attn(d, d->Hkv, Rp_doc, (long)n, true, kTargetWaves - loc_waves);
        }
        // Quadrature path at decode: the pairs' LDS-staged blocks and the local
        // part's, as LDS-staged blocks of one shape, in one launch of at most
        // one block per CU.  That launch is short (a few stages per block), and
        // 96-key stages at one block per CU serve it better than the 32-key
        // stages at two that stream the long document passes (1M-token
        // Quadrature path 19.2 us against 20.7-24.3 us).  The local part takes
        // its key stages as splits (at most two: a 384-key local part in 64
        // blocks of two stages leaves the pairs 148 blocks of three stages
        // instead of 112 of four beside 128 local blocks of one; 19.73 -> 19.12
        // us, and 21.5 us with one split), the pairs the remaining block slots.
        if (sp.kvp && !exact && sp.kvpl.lds && sp.kvpl.S > 0 && !sp.kvpl.xcd && d->splits <= 0 &&
            sp.loc.S > 0 && !sp.loc.lds && d->dtype == NECTAR_BF16 && d->d == 128 && sp.loc.Rp <= 64 &&
            sp.kvpl.Rp <= 64) {
            const LdsShape psh{4, 1, 96, lds_blocks_per_cu(96)};
            const long slots = kTargetBlocksLds * psh.BPC;
            const long lstages = cdiv(loc->T_loc, psh.SK);
            const long lblocks = (long)sp.loc.P * std::min(lstages, 2L);
            if (lblocks <= slots / 2) {
                const AttnPlan l2 = plan_attn(d, sp.loc.P, sp.loc.Rp, loc->T_loc, true, kTargetWaves, lblocks, &psh);
                const AttnPlan k2 = plan_attn(d, sp.kvpl.P, sp.kvpl.Rp, (long)m->p, true, kTargetWaves,
                                              slots - (long)l2.P * l2.RB * l2.SB, &psh);
                if (l2.lds && k2.lds && !l2.xcd && !k2.xcd) {
                    sp.loc = l2;
                    sp.kvpl = k2;
                    sp.kvp_pair = true;
                }
            }
        }
        // Nectar path at decode (the decode module beside the local part only):
        // the local part in blocks of two split waves (the block's other two
        // waves, a second row group that does not exist, end at once), so its
        // caches spread over more CUs beside the module's blocks
        if (sp.mlp && !exact && sp.mlpl.dec && d->dtype == NECTAR_BF16 && !sp.loc.lds && sp.loc.S > 0 &&
            sp.loc.RT == 1 && sp.loc.RG == 1 && sp.loc.WS == 4 && d->splits <= 0) {
            sp.loc.WR = 2;
            sp.loc.WS = 2;
            sp.loc.RB = 1;
            sp.loc.SB = (int)cdiv(sp.loc.S, 2);
        }
        size_t off = align256(attn_partial_bytes(d, sp.loc));
        if (exact) {
            sp.off_doc = off;
            off += align256(attn_partial_bytes(d, sp.doc));
        }
        if (m) {
            sp.off_mod = off;
            off += align256(sp.mlp ? mlp_partial_bytes(d, sp.mlpl) : attn_partial_bytes(d, sp.kvpl));
        }
        sp.bytes = off;
    } else {
        size_t sub = sp.loc.ws;
        if (exact && sp.doc.ws > sub) sub = sp.doc.ws;
        if (sp.mlp && sp.mlpl.ws > sub) sub = sp.mlpl.ws;
        if (sp.kvp && sp.kvpl.ws > sub) sub = sp.kvpl.ws;
        if (sp.deep && sp.deep_ws > sub) sub = sp.deep_ws;
        size_t off = align256(sub);
        sp.off_px = off;
        off += exact ? pair_bytes(d) : 0;
        sp.off_pm = off;
        off += m ? pair_bytes(d) : 0;
        sp.off_pl = off;
        off += pair_bytes(d);
        sp.off_po = off;
        off += exact && m ? align256((size_t)d->R * d->Hq * d->d * 4) : 0;
        sp.bytes = off;
    }
    return sp;
}

// Deferred-finish parameters of one attention plan writing into part
// (read-outs, then statistics).
static AttnParams attn_partial_params(const nectar_attn_desc *d, const AttnPlan &pl, const void *q, const void *k,
                                      const void *v, int64_t bstride, int64_t hstride, int64_t row, int B, int Tq,
                                      long T_kv, int causal, int q_offset, void *part) {
    AttnParams a{};
    a.q = q; a.k = k; a.v = v;
    a.kv_bstride = bstride; a.kv_hstride = hstride; a.kv_row = row;
    a.Hq = d->Hq; a.G = d->Hq / d->Hkv; a.Hkv = d->Hkv; a.Tq = Tq; a.B = B; a.Rp = pl.Rp;
    a.T_kv = (int)T_kv; a.causal = causal; a.q_offset = q_offset;
    a.sl2 = score_scale(d) * 1.4426950408889634f;
    a.P = pl.P; a.S = pl.S; a.chunk = pl.chunk; a.tiles = pl.tiles; a.RG = pl.RG;
    a.WR = pl.WR; a.WS = pl.WS; a.RB = pl.RB; a.SB = pl.SB;
    a.xcd_group = pl.xcd ? 1 : 0;
    a.defer = 1;
    a.part_O = (float *)part;
    a.part_ml = (float2 *)((char *)part + (size_t)pl.P * pl.SB * pl.Rp * d->d * 4);
    return a;
}

static hipError_t launch_plan(const nectar_attn_desc *d, const AttnPlan &pl, const AttnParams &a, hipStream_t st) {
    if (pl.S == 0) return hipSuccess;
    return pl.lds ? launch_attn_rows_lds(a, pl.sh, st) : launch_attn_partial(a, d->dtype, d->d, pl.RT, st);
}

// The register-direct bf16 kernel serves both plans in one launch when they
// use the same row tiling.
static bool pairable(const nectar_attn_desc *d, const AttnPlan &x, const AttnPlan &y) {
    return d->dtype == NECTAR_BF16 && x.S > 0 && y.S > 0 && !x.lds && !y.lds && x.RT == y.RT;
}

static MlpParams mlp_partial_params(const nectar_attn_desc *d, const MlpPlan &pl, const nectar_module *m,
                                    const void *q, void *part) {
    MlpParams a{};
    a.q = q; a.W1 = m->W1; a.W2t = m->W2t; a.Ws = m->Ws; a.ws2 = m->ws2;
    a.b1 = m->b1; a.bs = m->bs; a.b2 = m->b2; a.bs2 = m->bs2;
    a.Hq = d->Hq; a.G = d->Hq / d->Hkv; a.Hkv = d->Hkv; a.Rp = pl.Rp;
    a.Ht = m->Ht; a.Hs = m->Hs; a.act = m->act;
    a.S = pl.S; a.chunk_t = pl.ct; a.chunk_s = pl.cs; a.RG = pl.RG;
    a.WR = pl.WR; a.WS = pl.WS; a.RB = pl.RB; a.SB = pl.SB; a.nwt = pl.Wt; a.nws = pl.Ws;
    a.defer = 1;
    a.part_O = (float *)part;
    a.part_s = (float *)((char *)part + (size_t)d->Hkv * pl.SB * pl.Rp * d->d * 4);
    return a;
}

static bool exact_requested(const nectar_step_outputs *o) {
    return o->out_exact || o->lse_exact || o->alpha_out || o->A_out;
}

// Composed layer step: each document-side part finishes itself into its pair
// (the caller's pair outputs or scratch), the local pass merges one of them in
// place and a merge launch handles the second.
static hipError_t run_step_composed(const nectar_attn_desc *desc, const StepPlan &sp, int64_t n,
                                    const nectar_local_desc *loc, const void *q, const void *k, const void *v,
                                    const void *k_loc, const void *v_loc, const nectar_module *module,
                                    const nectar_step_outputs *outs, char *w, hipStream_t st) {
    const size_t lse_bytes = align256((size_t)desc->R * desc->Hq * 4);
    auto pair = [&](size_t off, float *lse, float *A, float **pl, float **pA) {
        *pl = lse ? lse : (float *)(w + off);
        *pA = A ? A : (float *)(w + off + lse_bytes);
    };
    struct Merge { const float *lse, *A; void *out; float *out_lse; };
    Merge mg[2];
    int nm = 0;
    hipError_t e = hipSuccess;
    if (sp.exact) {
        float *al, *Ax;
        pair(sp.off_px, outs->alpha_out, outs->A_out, &al, &Ax);
        CombineParams cp{};
        cp.lse_out = al; cp.A_out = Ax;
        e = run_attention(desc, sp.doc, q, k, v, 0, n * doc_row(desc), doc_row(desc), 1, desc->R, (long)n, 0, 0, cp,
                          w, st);
        if (outs->out_exact || outs->lse_exact) mg[nm++] = Merge{al, Ax, outs->out_exact, outs->lse_exact};
    }
    if (e == hipSuccess && module) {
        float *am, *Am;
        pair(sp.off_pm, outs->a_out, outs->Am_out, &am, &Am);
        if (sp.mlp) {
            e = run_mlp(desc, sp.mlpl, module, q, am, Am, w, st);
        } else if (sp.deep) {
            e = run_deep(desc, module->deep, q, am, Am, w, st);
        } else {
            CombineParams cp{};
            cp.lse_out = am; cp.A_out = Am;
            e = run_attention(desc, sp.kvpl, q, module->W, module->Z, 0, module->p * desc->d, desc->d, 1, desc->R,
                              (long)module->p, 0, 0, cp, w, st);
        }
        if (outs->out_nectar || outs->lse_nectar) mg[nm++] = Merge{am, Am, outs->out_nectar, outs->lse_nectar};
    }
    if (e != hipSuccess) return e;
    // local pass: its pair (requested, or needed by a second merge) and the first merge in place
    float *lam = outs->lam_out, *Aloc = outs->Aloc_out;
    if (nm == 2) pair(sp.off_pl, outs->lam_out, outs->Aloc_out, &lam, &Aloc);
    if (nm == 0 && !lam && !Aloc) return e;      // nothing needs the local part
    CombineParams cp{};
    cp.lse_out = lam; cp.A_out = Aloc;
    if (nm > 0) {
        cp.x_lse = mg[0].lse; cp.x_A = mg[0].A; cp.out = mg[0].out; cp.out_lse = mg[0].out_lse;
    }
    const int64_t hstride = (int64_t)loc->T_cap * desc->d;
    e = run_attention(desc, sp.loc, q, k_loc, v_loc, hstride * desc->Hkv, hstride, desc->d, loc->B, loc->Tq, loc->T_loc, 1,
                      loc->q_offset, cp, w, st);
    for (int i = 1; i < nm && e == hipSuccess; ++i) {
        // out may be NULL (only the merged log-normaliser requested): write the output to scratch
        MergeParams mp;
        mp.a = mg[i].lse; mp.A = mg[i].A; mp.lam = lam; mp.A_loc = Aloc;
        mp.out = mg[i].out ? mg[i].out : (void *)(w + sp.off_po);
        mp.lse_out = mg[i].out_lse;
        mp.rows = (long)desc->R * desc->Hq;
        e = launch_merge(mp, desc->dtype, desc->d, st);
    }
    return e;
}

// ---------------------------------------------------------------------------
// The exact document attention as its two passes.

size_t nectar_doc_attn_partials_size(const nectar_attn_desc *desc, int64_t n) {
    if (check_desc(desc) != NECTAR_OK || n < 0 || n > 0x7fffffffL - kTile) return 0;
    return attn_partial_bytes(desc, plan_doc(desc, (long)n));
}

nectar_status nectar_doc_attn_partials(const nectar_attn_desc *desc, int64_t n, const void *q, const void *k,
                                       const void *v, void *partials, size_t bytes, void *stream) {
    nectar_status s = check_desc(desc);
    if (s != NECTAR_OK) return s;
    if (n < 0) return NECTAR_EINVAL;
    if (n > 0x7fffffffL - kTile) return NECTAR_EUNSUPPORTED;
    if (desc->R == 0) return NECTAR_OK;
    if (!tensor_ok(q)) return NECTAR_EINVAL;
    if (n > 0 && (!tensor_ok(k) || !tensor_ok(v))) return NECTAR_EINVAL;
    const AttnPlan pl = plan_doc(desc, (long)n);
    if ((s = check_ws(attn_partial_bytes(desc, pl), partials, bytes)) != NECTAR_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    const AttnParams a = attn_partial_params(desc, pl, q, k, v, 0, n * doc_row(desc), doc_row(desc), 1, desc->R,
                                             (long)n, 0, 0, partials);
    return finish(launch_plan(desc, pl, a, st), st);
}

nectar_status nectar_doc_attn_combine(const nectar_attn_desc *desc, int64_t n, const void *partials, size_t bytes,
                                      float *alpha_out, float *A_out, void *stream) {
    nectar_status s = check_desc(desc);
    if (s != NECTAR_OK) return s;
    if (n < 0) return NECTAR_EINVAL;
    if (n > 0x7fffffffL - kTile) return NECTAR_EUNSUPPORTED;
    if (desc->R == 0) return NECTAR_OK;
    if (!f32_ok(alpha_out) || !rows_ok(A_out)) return NECTAR_EINVAL;
    const AttnPlan pl = plan_doc(desc, (long)n);
    const size_t need = attn_partial_bytes(desc, pl);
    if (bytes < need) return NECTAR_EWORKSPACE;
    if (need > 0 && (!partials || !aligned(partials, 16))) return NECTAR_EINVAL;
    CombineParams cp{};
    cp.lse_out = alpha_out; cp.A_out = A_out;
    cp.part_O = (const float *)partials;
    cp.part_ml = (const float2 *)((const char *)partials + (size_t)pl.P * pl.SB * pl.Rp * desc->d * 4);
    cp.Hq = desc->Hq; cp.G = desc->Hq / desc->Hkv; cp.Hkv = desc->Hkv; cp.Tq = desc->R;
    cp.P = desc->Hkv; cp.S = pl.S > 0 ? pl.SB : 0; cp.Rp = desc->R * (desc->Hq / desc->Hkv);
    hipStream_t st = (hipStream_t)stream;
    return finish(launch_attn_combine(cp, desc->dtype, desc->d, st), st);
}

size_t nectar_layer_step_workspace_size(const nectar_attn_desc *desc, int64_t n, const nectar_local_desc *loc,
                                        const nectar_module *module, int exact) {
    if (check_desc(desc) != NECTAR_OK || check_local(desc, loc) != NECTAR_OK) return 0;
    if (n < 0 || n > 0x7fffffffL - kTile) return 0;
    if (module && check_module(desc, module) != NECTAR_OK) return 0;
    return plan_step(desc, n, loc, module, exact != 0).bytes;
}

// Every argument check of the layer step (no HIP call); on NECTAR_OK *sp holds
// the plan, unless R == 0 (*noop: nothing to launch).
static nectar_status check_layer_step(const nectar_attn_desc *desc, int64_t n, const nectar_local_desc *loc,
                                      const void *q, const void *k, const void *v, const void *k_loc,
                                      const void *v_loc, const nectar_module *module,
                                      const nectar_step_outputs *outs, StepPlan *sp, bool *noop) {
    *noop = false;
    nectar_status s = check_desc(desc);
    if (s != NECTAR_OK) return s;
    if ((s = check_local(desc, loc)) != NECTAR_OK) return s;
    if (!outs) return NECTAR_EINVAL;
    if (module && (s = check_module(desc, module)) != NECTAR_OK) return s;
    const bool exact = exact_requested(outs);
    const bool nect = outs->out_nectar || outs->lse_nectar || outs->a_out || outs->Am_out;
    if (nect != (module != nullptr)) return NECTAR_EINVAL;
    if (!exact && !nect && !outs->lam_out && !outs->Aloc_out) return NECTAR_EINVAL;
    if (n < 0) return NECTAR_EINVAL;
    if (n > 0x7fffffffL - kTile) return NECTAR_EUNSUPPORTED;
    const float *f32s[] = {outs->lse_exact, outs->alpha_out, outs->lse_nectar, outs->a_out, outs->lam_out};
    for (const float *f : f32s)
        if (f && !f32_ok(f)) return NECTAR_EINVAL;
    const void *rows[] = {outs->A_out, outs->Am_out, outs->Aloc_out, outs->out_exact, outs->out_nectar};
    for (const void *r : rows)
        if (r && !rows_ok(r)) return NECTAR_EINVAL;
    if (desc->R == 0) {
        *noop = true;
        return NECTAR_OK;
    }
    if (!tensor_ok(q)) return NECTAR_EINVAL;
    if (loc->T_loc > 0 && (!tensor_ok(k_loc) || !tensor_ok(v_loc))) return NECTAR_EINVAL;
    if (exact && n > 0 && (!tensor_ok(k) || !tensor_ok(v))) return NECTAR_EINVAL;
    *sp = plan_step(desc, n, loc, module, exact);
    return NECTAR_OK;
}

// The launches of a checked layer step on workspace w (at least sp.bytes).
static hipError_t run_layer_step(const nectar_attn_desc *desc, const StepPlan &sp, int64_t n,
                                 const nectar_local_desc *loc, const void *q, const void *k, const void *v,
                                 const void *k_loc, const void *v_loc, const nectar_module *module,
                                 const nectar_step_outputs *outs, char *w, hipStream_t st) {
    if (!sp.fused) return run_step_composed(desc, sp, n, loc, q, k, v, k_loc, v_loc, module, outs, w, st);
    const int G = desc->Hq / desc->Hkv;
    FinishParams f{};
    f.Hq = desc->Hq; f.G = G; f.Hkv = desc->Hkv; f.Tq = loc->Tq;
    f.P = sp.loc.P; f.Rp = sp.loc.Rp; f.Rp_doc = desc->R * G;
    f.lam_out = outs->lam_out; f.Aloc_out = outs->Aloc_out;
    hipError_t e = hipSuccess;
    const int64_t hstride = (int64_t)loc->T_cap * desc->d;
    const AttnParams ap_loc = attn_partial_params(desc, sp.loc, q, k_loc, v_loc, hstride * desc->Hkv, hstride, desc->d,
                                                  loc->B, loc->Tq, loc->T_loc, 1, loc->q_offset, w);
    bool loc_done = false, mod_done = false;
    const AttnParams ap_doc = attn_partial_params(desc, sp.doc, q, k, v, 0, n * doc_row(desc), doc_row(desc), 1,
                                                  desc->R, (long)n, 0, 0, w + sp.off_doc);
    MlpParams mp{};
    if (sp.mlp) mp = mlp_partial_params(desc, sp.mlpl, module, q, w + sp.off_mod);
    // decode shapes: the attention blocks and the module's blocks in one launch
    const bool mlp_dec = sp.mlp && !sp.mlpl.prefill && desc->dtype == NECTAR_BF16;
    if (mlp_dec && sp.mlpl.RT == 1 && sp.exact && pairable(desc, sp.doc, sp.loc) && sp.doc.RT == 1) {
        e = launch_step_partials(ap_doc, &ap_loc, mp, desc->d, 1, st);
        loc_done = mod_done = true;
    } else if (mlp_dec && !sp.exact && sp.loc.S > 0 && !sp.loc.lds && sp.loc.RT == 1) {
        e = launch_step_partials(ap_loc, nullptr, mp, desc->d, sp.mlpl.RT, st);
        loc_done = mod_done = true;
    }
    if (sp.exact) {
        if (loc_done) {
            // already launched with the local and module blocks
        } else if (pairable(desc, sp.doc, sp.loc)) {
            e = launch_attn_partial_pair(ap_doc, ap_loc, desc->d, sp.doc.RT, st);
            loc_done = true;
        } else {
            e = launch_plan(desc, sp.doc, ap_doc, st);
        }
        FinishSet &x = f.set[f.nsets++];
        x.S = sp.doc.S > 0 ? sp.doc.SB : 0;
        x.O = (const float *)(w + sp.off_doc);
        x.ml = (const float2 *)(w + sp.off_doc + (size_t)sp.doc.P * sp.doc.SB * sp.doc.Rp * desc->d * 4);
        x.lse_out = outs->alpha_out; x.A_out = outs->A_out; x.out = outs->out_exact; x.out_lse = outs->lse_exact;
    }
    if (e == hipSuccess && module) {
        FinishSet &x = f.set[f.nsets++];
        x.O = (const float *)(w + sp.off_mod);
        x.lse_out = outs->a_out; x.A_out = outs->Am_out; x.out = outs->out_nectar; x.out_lse = outs->lse_nectar;
        if (sp.mlp) {
            if (!mod_done)
                e = sp.mlpl.dec ? launch_mlp_decode(mp, desc->d, sp.mlpl.RT, st)
                                : sp.mlpl.lds32 ? launch_mlp_rows_lds32(mp, st)
                                                : (sp.mlpl.prefill ? launch_mlp_prefill(mp, st)
                                                                   : launch_mlp_partial(mp, desc->dtype, desc->d,
                                                                                        sp.mlpl.RT, st));
            x.S = sp.mlpl.SB;
            x.s = (const float *)(w + sp.off_mod + (size_t)desc->Hkv * sp.mlpl.SB * sp.mlpl.Rp * desc->d * 4);
            x.b2 = module->b2; x.bs2 = module->bs2;
        } else {
            const AttnParams ap_kvp = attn_partial_params(desc, sp.kvpl, q, module->W, module->Z, 0,
                                                          module->p * desc->d, desc->d, 1, desc->R, (long)module->p,
                                                          0, 0, w + sp.off_mod);
            if (sp.kvp_pair) {
                e = launch_attn_rows_lds_pair(ap_kvp, ap_loc, sp.kvpl.sh, st);
                loc_done = true;
            } else {
                e = launch_plan(desc, sp.kvpl, ap_kvp, st);
            }
            x.S = sp.kvpl.S > 0 ? sp.kvpl.SB : 0;
            x.ml = (const float2 *)(w + sp.off_mod + (size_t)sp.kvpl.P * sp.kvpl.SB * sp.kvpl.Rp * desc->d * 4);
        }
    }
    if (e == hipSuccess) {
        if (!loc_done) e = launch_plan(desc, sp.loc, ap_loc, st);
        f.S_loc = sp.loc.S > 0 ? sp.loc.SB : 0;
        f.loc_O = (const float *)w;
        f.loc_ml = (const float2 *)(w + (size_t)sp.loc.P * sp.loc.SB * sp.loc.Rp * desc->d * 4);
    }
    if (e == hipSuccess) e = launch_finish(f, desc->dtype, desc->d, st);
    return e;
}

nectar_status nectar_layer_step(const nectar_attn_desc *desc, int64_t n, const nectar_local_desc *loc,
                                const void *q, const void *k, const void *v, const void *k_loc,
                                const void *v_loc, const nectar_module *module,
                                const nectar_step_outputs *outs, void *ws, size_t ws_bytes, void *stream) {
    StepPlan sp;
    bool noop;
    nectar_status s = check_layer_step(desc, n, loc, q, k, v, k_loc, v_loc, module, outs, &sp, &noop);
    if (s != NECTAR_OK || noop) return s;
    if ((s = check_ws(sp.bytes, ws, ws_bytes)) != NECTAR_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    return finish(run_layer_step(desc, sp, n, loc, q, k, v, k_loc, v_loc, module, outs, (char *)ws, st), st);
}

// Device address of `scratch` on the device of `stream` (the current device for
// the null stream), looked up once per device with that device current.
static nectar_status static_scratch(hipStream_t st, char **out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *ptr[kMaxDevices] = {};
    int cur = -1, dev = -1;
    if (hipGetDevice(&cur) != hipSuccess) return NECTAR_EHIP;
    dev = cur;
    if (st && hipStreamGetDevice(st, &dev) != hipSuccess) return NECTAR_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return NECTAR_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return NECTAR_EHIP;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess) return NECTAR_EHIP;
        if (e != hipSuccess || !p) return NECTAR_EHIP;
        ptr[dev] = p;
    }
    *out = (char *)ptr[dev];
    return NECTAR_OK;
}

nectar_status nectar_layer_step_static(const nectar_attn_desc *desc, int64_t n, const nectar_local_desc *loc,
                                       const void *q, const void *k, const void *v, const void *k_loc,
                                       const void *v_loc, const nectar_module *module,
                                       const nectar_step_outputs *outs, void *stream) {
    StepPlan sp;
    bool noop;
    nectar_status s = check_layer_step(desc, n, loc, q, k, v, k_loc, v_loc, module, outs, &sp, &noop);
    if (s != NECTAR_OK || noop) return s;
    if (sp.bytes > (size_t)NECTAR_STATIC_SCRATCH_BYTES) return NECTAR_EWORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    char *w = nullptr;
    if (sp.bytes > 0 && (s = static_scratch(st, &w)) != NECTAR_OK) return s;
    return finish(run_layer_step(desc, sp, n, loc, q, k, v, k_loc, v_loc, module, outs, w, st), st);
}

}  // extern "C"
