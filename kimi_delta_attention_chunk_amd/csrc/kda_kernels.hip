// kda_kernels.hip -- gfx950 (MI355X, CDNA4) kernels and C ABI of the KDA chunked forward.
//
// Method (FlashKDA README, section 功能说明, chunk equations): inside a chunk of n <= 64 tokens
// with running gate sums G (restarted every chunk),
//     Kt = exp(G)*K,  Kb = exp(-G)*K,  Qt = scale*exp(G)*Q,
//     T = strictly-lower(diag(beta) Kt Kb^T),  Ainv = (I + T)^-1,
//     U = Ainv diag(beta) V,  W = Ainv diag(beta) Kt,
// and the state is carried from chunk to chunk.  The carry used here (the plain reading; the
// vLLM #43195 summary, sections 实现拆解 and 关键源码片段, names the same per-chunk products
// h and v_new and an output kernel o = q h + A v_new):
//     V_new = U - W S^T,   O = Qt S^T + Aqk V_new,   Aqk = lower-with-diagonal(Qt Kb^T),
//     S <- S diag(exp(G_last)) + V_new^T (K * exp(G_last - G)).
// Kernels:
//   kda_intra_kernel  one workgroup per (64-token chunk, value head), fully parallel.  Computes
//                     the log2-space running gate sum, the decayed operands, T and Aqk on MFMA
//                     (diagonal blocks bf16, T's as hi/lo pairs; blocks below the diagonal
//                     fp16), the fp32 blocked inverse, W and U, and folds the chunk-local terms:
//                     Q' = Qt - Aqk W and O_intra = Aqk U, so that O = Q' S^T + O_intra.
//                     Writes W, Q', K_dec, U, O_intra and gamma_last in MFMA fragment order.
//   kda_scan_kernel   one workgroup per (sequence, value head, Dv tiles) walks the chunks in
//                     order with its state tiles resident in registers:
//                     V_new = U - W S^T, O = Q' S^T + O_intra, S <- gamma*S + K_dec^T V_new.
//   When few (sequence, head) chains would leave most compute units idle, the two-level scan
//   replaces kda_scan_kernel: kda_seg_kernel walks every segment of a sequence at once (from a
//   zero state and from identity rows), kda_combine_kernel chains the segment entry states, and
//   kda_out_kernel completes the outputs of every segment after the first in parallel.
//
// Overflow safety (vLLM #43195 summary, 实现拆解 / 关键源码片段: gates kept in log2 space and
// every decay an exp2 of a difference; flash-linear-attention PR #656: 16-token sub-blocks).
// exp(-G) is never formed.  For sub-blocks I > J the decay between rows i (block I) and j
// (block J) is split at the first row r_I of block I into two factors <= 1; inside a diagonal
// block the read key carries 2^(G_r - G_j) <= 2^(15 * 5 * log2 e) < 2^109 for g >= -5, finite
// in fp32/bf16 (so the diagonal blocks stay in bf16; the factors <= 1 of the other blocks fit
// fp16), and masked entries are removed by select, never by multiplication.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "kda.h"
#include "kda_plan.h"

namespace kda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

struct Params {
    const __bf16* q;
    const __bf16* k;
    const __bf16* v;
    const float* g;
    const __bf16* graw;      // raw bf16 gate (gate mode 2), v's layout
    const float* a_log;      // [n_v]     gate mode 2
    const float* dt_bias;    // [n_v, D]  gate mode 2
    float lower_bound;       //           gate mode 2
    const __bf16* beta;
    const float* init;
    const int32_t* cu;
    __bf16* out;
    float* fin;
    _Float16* Wf; // [record][tt 4][kb 4][lane 64][8]         W[16tt+m][32kb+8q+j] (fp16)
    _Float16* Qf; // [record][tt 4][kb 4][lane 64][8]         Q'[16tt+m][32kb+8q+j] (fp16)
    _Float16* Kf; // [record][mt 8][s 2][lane 64][8]          K_dec[32s+8q+j][16mt+m] (fp16)
    _Float16* Uf; // [record][nt 8][tt 4][lane 64][4]         U[16tt+4q+i][16nt+n] (fp16)
    __bf16* Of;   // [record][nt 8][tt 4][lane 64][4]         O_intra[16tt+n][16nt+4q+i]
    float* Gf;    // [record][128]                            2^(G2_last)
    // two-level scan, per (sequence*head, segment) and per record, in MFMA fragment order:
    _Float16* Pt; // [M 8][kb 4][lane 64][8]         P_s[32kb+8q+j][16M+m]      transfer matrix (fp16)
    float* Nst;   // [t 8][M 8][lane 64][4]          N_s[16t+m][16M+4q+i]       zero-start end state
    __bf16* Sin;  // [t 8][kb 4][lane 64][8]         S_in[16t+m][32kb+8q+j]     entry state
    __bf16* O0;   // [t 8][tt 4][lane 64][4]         O0[16tt+m][16t+4q+i]       zero-start outputs
    __bf16* Rf;   // [tt 4][kb 4][lane 64][8]        R[16tt+m][32kb+8q+j]       R = Q' P^T
    int layout, batch, seq_len, n_qk, n_v, group, nc_max;
    int scan_tiles;
    int seg_p;     // segments per sequence of the two-level scan (1 = one level)
    int intra_units;   // intra kernel: records / group (chunk slot, q/k head) units
    float scale;
    uint32_t flags;
};

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi): about 16 mantissa bits in two MFMA
// operands; a product of two such pairs drops only the lo*lo term.
__device__ __forceinline__ __bf16 bf16_lo(float x, __bf16 hi) { return (__bf16)(x - (float)hi); }
// Stores into one workgroup's share of a workspace array at device scope (cache policy sc1):
// they are written through the L2, so the kernel's end does not wait for a write-back of every
// dirty record line, and the next kernel, on any XCD, reads them from the memory-side cache.
// Raw buffer stores: the hardware drops any store past `bytes`.
struct DevStore {
    __amdgpu_buffer_rsrc_t r;
    static constexpr int kDevScope = 16;   // sc1
    __device__ __forceinline__ DevStore(void* base, unsigned bytes)
        : r(__builtin_amdgcn_make_buffer_rsrc(base, 0, int(bytes), 0x00020000)) {}
    template <typename T>
    __device__ __forceinline__ void put(unsigned byte_off, const T& v) const {
        if constexpr (sizeof(T) == 16)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, int(byte_off), 0,
                                                   kDevScope);
        else if constexpr (sizeof(T) == 8)
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, int(byte_off), 0,
                                                  kDevScope);
        else
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, int(byte_off), 0,
                                                  kDevScope);
    }
};

// Buffer load from a wave-uniform base (scalar resource) at a per-lane byte offset: no 64-bit
// per-lane address is formed per chunk, so a loop of chunk loads keeps no address registers
// that alias the loaded data.
template <typename T>
__device__ __forceinline__ T buf_load(const void* base, unsigned bytes, unsigned byte_off) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
    if constexpr (sizeof(T) == 16)
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, int(byte_off), 0, 0));
    else if constexpr (sizeof(T) == 8)
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, int(byte_off), 0, 0));
    else
        return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(r, int(byte_off), 0, 0));
}

// Chunk operand load: a buffer load (scalar base, no per-chunk 64-bit lane address) for the
// one-tile prefetched scan, where it was measured faster; a plain load elsewhere.
template <bool BUF, typename T>
__device__ __forceinline__ T ld_op(const void* base, unsigned bytes, unsigned byte_off) {
    if constexpr (BUF) return buf_load<T>(base, bytes, byte_off);
    else return *reinterpret_cast<const T*>(static_cast<const char*>(base) + byte_off);
}

#define SPLIT_BF16(x, hi, lo)          \
    do {                               \
        const float x_ = (x);          \
        (hi) = (__bf16)x_;             \
        (lo) = bf16_lo(x_, (hi));      \
    } while (0)

// LDS-only barrier: waits for this wave's LDS traffic, then the workgroup barrier.  Outstanding
// global loads (prefetches) stay in flight.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Orders this wave's LDS accesses (a wave's LDS operations complete in issue order; the
// compiler must not move accesses across this point).
__device__ __forceinline__ void wave_lds_fence() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Sequence geometry: valid length and the chunk-slot base, identical in both kernels.
__device__ __forceinline__ void seq_info(const Params& p, int b, int& c0, int& len,
                                         int& slot0) {
    if (p.layout == KDA_LAYOUT_TND) {
        int a = p.cu[b], e = p.cu[b + 1];
        a = a < 0 ? 0 : (a > p.seq_len ? p.seq_len : a);
        e = e < a ? a : (e > p.seq_len ? p.seq_len : e);
        c0 = a;
        len = e - a;
        slot0 = a / kChunk + b;
    } else {
        int l = p.seq_len;
        if (p.cu) {
            l = p.cu[b + 1] - p.cu[b];
            l = l < 0 ? 0 : (l > p.seq_len ? p.seq_len : l);
        }
        c0 = 0;
        len = l;
        slot0 = b * p.nc_max;
    }
}

// Sequence of a chunk slot: the last b whose first slot is <= slot (TND), or slot / nc_max.
__device__ __forceinline__ int slot_batch(const Params& p, int slot) {
    if (p.layout != KDA_LAYOUT_TND) return int(unsigned(slot) / unsigned(p.nc_max));
    int lo = 0, hi = p.batch - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        int cm = p.cu[mid];
        cm = cm < 0 ? 0 : (cm > p.seq_len ? p.seq_len : cm);
        if (cm / kChunk + mid <= slot) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Element offset of token 0 and the token stride for (sequence b, head h) of a tensor with
// `heads` heads and `e` elements per (token, head): BNSD [B,H,S,e], BSND [B,S,H,e], TND [T,H,e].
__device__ __forceinline__ void row_geom(const Params& p, int b, int h, int heads, int e,
                                         int c0, size_t& base, size_t& stride) {
    if (p.layout == KDA_LAYOUT_BNSD) {
        base = (size_t(b) * heads + h) * size_t(p.seq_len) * e;
        stride = size_t(e);
    } else if (p.layout == KDA_LAYOUT_BSND) {
        base = (size_t(b) * p.seq_len * heads + h) * size_t(e);
        stride = size_t(heads) * e;
    } else {
        base = (size_t(c0) * heads + h) * size_t(e);
        stride = size_t(heads) * e;
    }
}

// ---------------------------------------------------------------------------------------------
// Intra-chunk kernel
// ---------------------------------------------------------------------------------------------
//
// One workgroup of four waves per (64-token chunk, value head); wave w owns token block I = w
// (tokens 16I .. 16I+15).  Lane (q4, n16) holds token 16I + n16 and channels 32kb + 8q4 + e
// (kb < D/32, e < 8) of q, k, v and g, loaded straight from HBM in this "row layout", which
// is at once the A operand of an MFMA over channels and its B operand with tokens as columns.
//
// Products over tokens (W, U, O_intra, Q') need operands with eight consecutive tokens per
// lane.  Those are made exactly on the MFMA unit: a row-layout fragment times a 0/1 selection
// matrix returns, in the accumulator layout, four consecutive tokens of one channel per lane
// (bf16 inputs, fp32 sums of one nonzero term: no rounding).  Lanes then store 8-byte pieces
// into token-grouped LDS tiles that the consumers read back with 16-byte loads.
//
// The workgroup keeps its LDS under 80 KB and its registers under 256 per lane, so two
// workgroups share a compute unit and one's memory phase overlaps the other's arithmetic; at
// head dim 64 under 53 KB and 168 registers, so three do.  When the whole grid is resident at
// once, an eight-wave form (two waves per token block, each with half the channels) shortens
// the workgroup's latency instead.

constexpr int BLK_LD = 20;              // fp32 row stride of a stored 16 x 16 block
constexpr int BLK_SZ = 16 * BLK_LD;     // floats per stored block
constexpr int N_BLK = 10;               // lower-triangular 16 x 16 blocks of a 64 x 64 matrix
constexpr int TILE = 8 * 16 * 8 * 2;    // one token-grouped tile [group 8][n16][8] bf16: 2 KB

// LDS of the intra kernel for head dim D:
//   Aqk blocks (12800) | Ainv blocks (12800) | beta[64] (256) | region X | vecA[4][128] fp32
// The Ainv region holds, until the inverse is formed, the per-channel factor rows
//   vec: BV[6][128], C[4][128] fp32 (5120) at Ainv + 0;
// vecA, the factor rows of Q~ and K~, has its own 2048 bytes, so that the operands made from it
// can be formed while the inverse writes its blocks.
// Region X, by phase:
//   gate sums      first[4][128], dlast[4][128] fp32 (4096)                  at X + 0
//   T/Aqk          sR [pair 6][kb D/32][lane 64] f16x8 (6 D/32 KB)            at X + 0
//                  sT blocks (12800)                                          at X + X_T
//   inverse        sTmp [wave 4][16][BLK_LD] fp32 (5120)                      at X + 0
//   W, U           sKt hi/lo tiles (2 D/16 tiles), sVt (D/16 tiles)           at X + 0
//   O_intra, Q'    sW (-W, D/16 tiles), sU (D/16 tiles)                       at X + 0
// D = 128: 77,056 B (two workgroups per compute unit); D = 64: 52,992 B (three).  The eight-wave
// form (HV = 2) also keeps, through phases 1 and 2, the half sums of squares [2][64][2] fp32 and
// the second channel half's T products [block 10][lane 64][4] fp32 after the T blocks.
template <int D, int HV = 1>
struct IntraLds {
    static constexpr int OFF_AQK = 0;
    static constexpr int OFF_AI = OFF_AQK + N_BLK * BLK_SZ * 4;
    static constexpr int OFF_BETA = OFF_AI + N_BLK * BLK_SZ * 4;
    static constexpr int OFF_X = OFF_BETA + 256;
    static constexpr int AI_VEC = 0;
    static constexpr int TILES = D / 16;
    static constexpr int X_R = 0;
    static constexpr int X_T = 6 * (D / 32) * 64 * 16;
    static constexpr int X_TMP = 0;
    static constexpr int X_KT = 0;
    static constexpr int X_KTL = TILES * TILE;
    static constexpr int X_VT = 2 * TILES * TILE;
    static constexpr int X_W = 0;
    static constexpr int X_U = TILES * TILE;
    static constexpr int X_NRM = X_T + N_BLK * BLK_SZ * 4;   // eight waves: half sums [2][64][2]
    static constexpr int X_TP = X_NRM + 1024;                  // eight waves: T half products
    static constexpr int X_P2 = HV == 2 ? X_TP + N_BLK * 1024 : X_NRM;   // end of phase 1-2 use
    static constexpr int X_BYTES = X_P2 > 3 * TILES * TILE ? X_P2 : 3 * TILES * TILE;
    static constexpr int OFF_VECA = OFF_X + X_BYTES;   // factor rows vecA[4][128] fp32
    static constexpr int BYTES = OFF_VECA + 2048;
    // workgroups per compute unit; as the launch bound it caps the registers: the eight-wave form
    // must fit 128 so that two of its workgroups share a compute unit
    static constexpr int PER_CU = (D == 64 && HV == 1) ? 3 : 2;
    static_assert(5120 <= N_BLK * BLK_SZ * 4, "factor rows fit the Ainv region");
    static_assert(X_BYTES >= 4096 && X_BYTES >= 4 * BLK_SZ * 4, "gate sums and staging fit X");
    static_assert(X_TMP + 4 * BLK_SZ * 4 <= X_T, "inverse staging ends before the T blocks");
    static_assert(PER_CU * BYTES <= 160 * 1024, "the workgroups of one compute unit fit its LDS");
};

// vector rows inside vec (the Ainv region until the inverse), 128 floats each
constexpr int VEC_BV = 0;   // 6 rows: exp(G[16I] - G[16J]) for (I,J) = (1,0),(2,0),(2,1),(3,0),(3,1),(3,2)
constexpr int VEC_C = 6;    // 4 rows: exp(G_last - G[16I])

__device__ __forceinline__ int pair_index(int I, int J) {  // I > J
    return (I * (I - 1)) / 2 + J;
}
__device__ __forceinline__ int blk(int I, int J) {         // I >= J
    return (I * (I + 1)) / 2 + J;
}

// Inclusive prefix sum over the 16 lanes of a DPP row (lanes 16r .. 16r+15).
__device__ __forceinline__ float row_scan16(float x) {
#define KDA_ROW_SHR(v, ctrl) \
    __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, 0xf, 0xf, true))
    x += KDA_ROW_SHR(x, 0x111);
    x += KDA_ROW_SHR(x, 0x112);
    x += KDA_ROW_SHR(x, 0x114);
    x += KDA_ROW_SHR(x, 0x118);
#undef KDA_ROW_SHR
    return x;
}

// 0/1 selection fragments (B operands).  With A a row-layout fragment of K-step kb,
//   sel_nat(h): C[token][n] = X[token][32kb + 16h + n]                   (channel tile 2kb+h)
//   sel_phi(h): C[token][n] = X[token][32kb + 8(n>>2) + 4h + (n&3)]       (tile 2kb+h, phi order)
// The phi order makes the accumulator rows 4q4 + r of tile (kb, h) the lane's own channels
// 32kb + 8q4 + 4h + r, so an accumulator initialised from row-layout registers lines up.
// Eight 16-bit elements, element t holding `bits` and the others zero (all zero when t lies
// outside [0, 8)): four selects instead of eight compares, eight selects and four packs.
__device__ __forceinline__ bf16x8 onehot8(int t, unsigned bits) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const unsigned v = bits << ((unsigned(t) & 1u) * 16u);
    const unsigned d = unsigned(t) >> 1;
    u32x4 r;
    r.x = d == 0u ? v : 0u;
    r.y = d == 1u ? v : 0u;
    r.z = d == 2u ? v : 0u;
    r.w = d == 3u ? v : 0u;
    return __builtin_bit_cast(bf16x8, r);
}
__device__ __forceinline__ bf16x8 sel_nat(int h, int q4, int n16) {
    return onehot8(16 * h + n16 - 8 * q4, 0x3F80u);   // bf16 1
}
__device__ __forceinline__ f16x8 sel_nat16(int h, int q4, int n16) {
    return __builtin_bit_cast(f16x8, onehot8(16 * h + n16 - 8 * q4, 0x3C00u));   // fp16 1
}
// negative: -1 in place of 1
__device__ __forceinline__ bf16x8 sel_phi(int h, int q4, int n16, bool negative = false) {
    return onehot8(q4 == (n16 >> 2) ? 4 * h + (n16 & 3) : -1, negative ? 0xBF80u : 0x3F80u);
}

__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) {
    bf16x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (__bf16)x[i];
    return r;
}
__device__ __forceinline__ f16x4 to_f16x4(f32x4 x) {
    f16x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (_Float16)x[i];
    return r;
}

// Token-grouped tile [tile 8][group 8][n16 16][8] bf16: group g holds tokens 8g .. 8g+7.  The
// accumulator lane (q4, n16) of token block I holds tokens 16I + 4q4 .. +3, i.e. half of group
// 2I + (q4 >> 1).
__device__ __forceinline__ void tile_put(__bf16* tile, int t, int I, int q4, int n16, bf16x4 v) {
    *reinterpret_cast<bf16x4*>(tile + ((t * 8 + 2 * I + (q4 >> 1)) * 16 + n16) * 8 + 4 * (q4 & 1)) = v;
}
__device__ __forceinline__ bf16x8 tile_get(const __bf16* tile, int t, int g, int n16) {
    return *reinterpret_cast<const bf16x8*>(tile + ((t * 8 + g) * 16 + n16) * 8);
}

// Eight consecutive fp32 entries of row n16 of a stored lower-triangular 64 x 64 matrix, row
// block I, columns 32s + 8q4 .. +7 (zero above the block diagonal).
__device__ __forceinline__ void blk_row8(const float* m, int I, int s, int q4, int n16, float (&x)[8]) {
    const int J = 2 * s + (q4 >> 1);
    if (J <= I) {
        const float* src = m + blk(I, J) * BLK_SZ + n16 * BLK_LD + 8 * (q4 & 1);
        const f32x4 a = *reinterpret_cast<const f32x4*>(src);
        const f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = a[e];
            x[4 + e] = b[e];
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
}

// GM: gate mode.  0: one fp32 natural-log decay per (token, key channel); 1: one per (token,
// value head) (KDA_SCALAR_GATE), broadcast over the key channels; 2: the raw bf16 gate per
// (token, key channel), activated at load as lower_bound * sigmoid(exp(A_log[h]) * (g_raw +
// dt_bias[h, c])) (KDA_RAW_GATE).
// D: head dim (d_k = d_v), 128 or 64.
// HV: waves per 16-token block.  With HV = 2 (eight waves) wave w owns token block I = w >> 1
// and channel half hc = w & 1: its loads, gate sums, decayed operands and transposes cover
// channels [hc D/2, (hc+1) D/2), its W, Q' tiles are the Dk tiles of that half and its U,
// O_intra tiles the Dv tiles of the same index range; the T/Aqk products over channels are
// summed from the two halves through LDS.
template <int GM, int D, int HV>
__global__ __launch_bounds__(kThreads * HV, (IntraLds<D, HV>::PER_CU * HV)) void kda_intra_kernel(Params p) {
    constexpr bool SG = GM == 1;
    constexpr int KB = D / 32;    // 32-channel K steps of a product over channels
    constexpr int NTD = D / 16;   // 16-wide channel (or Dv) tiles
    constexpr int KBW = KB / HV;  // channel blocks of this wave
    constexpr int NTW = NTD / HV; // W/Q' (Dk) and U/O_intra (Dv) tiles of this wave
    static_assert(HV == 1 || HV == 2, "one or two waves per token block");
    using LY = IntraLds<D, HV>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[LY::BYTES];
    float* sAqk = reinterpret_cast<float*>(smem + LY::OFF_AQK);
    float* sAi = reinterpret_cast<float*>(smem + LY::OFF_AI);
    float* sBeta = reinterpret_cast<float*>(smem + LY::OFF_BETA);
    float* sVec = reinterpret_cast<float*>(smem + LY::OFF_AI + LY::AI_VEC);
    float* sVecA = reinterpret_cast<float*>(smem + LY::OFF_VECA);
    unsigned char* X = smem + LY::OFF_X;
    float* sFirst = reinterpret_cast<float*>(X);               // [4][128]
    float* sDlast = sFirst + 512;                              // [4][128]
    f16x8* sR = reinterpret_cast<f16x8*>(X + LY::X_R);         // [pair 6][kb KB][lane 64]
    float* sT = reinterpret_cast<float*>(X + LY::X_T);
    float* sNrm = reinterpret_cast<float*>(X + LY::X_NRM);     // [half 2][token 64][q, k]
    float* sTp = reinterpret_cast<float*>(X + LY::X_TP);       // [block 10][lane 64][4]
    float* sTmp = reinterpret_cast<float*>(X + LY::X_TMP);
    __bf16* sKtH = reinterpret_cast<__bf16*>(X + LY::X_KT);
    __bf16* sKtL = reinterpret_cast<__bf16*>(X + LY::X_KTL);
    __bf16* sVt = reinterpret_cast<__bf16*>(X + LY::X_VT);
    __bf16* sW = reinterpret_cast<__bf16*>(X + LY::X_W);
    __bf16* sU = reinterpret_cast<__bf16*>(X + LY::X_U);

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar block indices
    const int lane = tid & 63;
    const int q4 = lane >> 4;
    const int n16 = lane & 15;
    const int I = HV == 2 ? (w >> 1) : w;     // token block
    const int hc = HV == 2 ? (w & 1) : 0;     // channel half
    const int kb0 = hc * KBW;                 // first channel block of this wave
    const int tw0 = hc * NTW;                 // first W/Q' and U/O_intra tile of this wave

    // Record rec = slot * n_v + h = unit * group + m, unit = slot * n_qk + hq.  With GQA the
    // group value heads of a unit (one chunk of one q/k head) run on one XCD, dispatched one
    // after another, so its L2 fetches that q/k chunk once: workgroup 8 r + x takes unit
    // (r / group) 8 + x, member r mod group (the identity without GQA).
    // (unsigned 32-bit arithmetic throughout: records and slots stay below 2^31, the plan
    // rejects larger grids, and a 64-bit or signed division costs the prologue that delays
    // every load of the workgroup)
    const unsigned pid = blockIdx.x;
    const unsigned gr = unsigned(p.group);
    const unsigned rr = pid >> 3;
    const unsigned rq = rr / gr;
    const unsigned unit = rq * 8u + (pid & 7u);
    if (unit >= unsigned(p.intra_units)) return;   // grid padding
    const unsigned rec32 = unit * gr + (rr - rq * gr);
    const unsigned slot_u = rec32 / unsigned(p.n_v);
    const int64_t rec = rec32;
    const int slot = int(slot_u);
    const int h = int(rec32 - slot_u * unsigned(p.n_v));
    const int hq = int(unsigned(h) / gr);

    // chunk slot -> (sequence b, chunk j)
    const int b = slot_batch(p, slot);
    int c0, len, slot0;
    seq_info(p, b, c0, len, slot0);
    const int j = slot - slot0;
    if (j < 0 || j * kChunk >= len) return;  // an unused slot: nothing reads it
    const int t0 = j * kChunk;
    const int n = (len - t0) < kChunk ? (len - t0) : kChunk;

    size_t qb, qs, vb, vs, bb, bs;
    row_geom(p, b, hq, p.n_qk, D, c0, qb, qs);
    row_geom(p, b, h, p.n_v, D, c0, vb, vs);
    row_geom(p, b, h, p.n_v, 1, c0, bb, bs);
    qb += size_t(t0) * qs;
    vb += size_t(t0) * vs;
    bb += size_t(t0) * bs;

    const int tok = 16 * I + n16;        // this lane's token inside the chunk
    const bool tv = tok < n;
    const int tc = tv ? tok : n - 1;     // rows past the tail are read clamped, then zeroed

    // ---- phase 0: every global load of the workgroup, in row layout --------------------------
    // The gate first (the prefix scan needs it first), then q, k, v and beta.  Rows past the
    // tail are read clamped and masked where they are consumed, so that no register written
    // here is rewritten before its load returns (which would make the wave wait for it).
    bf16x8 xq[KBW], xk[KBW], xv[KBW];
    f32x4 xg[2 * KBW];   // the fp32 gate, or (gate mode 2) dt_bias of the lane's channels
    bf16x8 xgr[KBW];     // gate mode 2: the raw gate
    float gsv;   // the one gate of this token with KDA_SCALAR_GATE (beta's layout)
    float alog = 0.f;
    float braw;
    if constexpr (SG) {
        gsv = p.g[bb + size_t(tc) * bs];
    } else if constexpr (GM == 2) {
        const __bf16* gr = p.graw + vb + size_t(tc) * vs;
        const float* db = p.dt_bias + size_t(h) * D;
#pragma unroll
        for (int i = 0; i < KBW; ++i) {
            const int c = 32 * (kb0 + i) + 8 * q4;
            xgr[i] = *reinterpret_cast<const bf16x8*>(gr + c);
            xg[2 * i] = *reinterpret_cast<const f32x4*>(db + c);
            xg[2 * i + 1] = *reinterpret_cast<const f32x4*>(db + c + 4);
        }
        alog = p.a_log[h];
    } else {
        const float* gr = p.g + vb + size_t(tc) * vs;
#pragma unroll
        for (int i = 0; i < KBW; ++i) {
            const int c = 32 * (kb0 + i) + 8 * q4;
            xg[2 * i] = *reinterpret_cast<const f32x4*>(gr + c);
            xg[2 * i + 1] = *reinterpret_cast<const f32x4*>(gr + c + 4);
        }
    }
    {
        const __bf16* qr = p.q + qb + size_t(tc) * qs;
        const __bf16* kr = p.k + qb + size_t(tc) * qs;
        const __bf16* vr = p.v + vb + size_t(tc) * vs;
#pragma unroll
        for (int i = 0; i < KBW; ++i) {
            const int c = 32 * (kb0 + i) + 8 * q4;
            xk[i] = *reinterpret_cast<const bf16x8*>(kr + c);
            xq[i] = *reinterpret_cast<const bf16x8*>(qr + c);
        }
#pragma unroll
        for (int i = 0; i < KBW; ++i)
            xv[i] = *reinterpret_cast<const bf16x8*>(vr + 32 * (kb0 + i) + 8 * q4);
        braw = (float)p.beta[bb + size_t(tc) * bs];
    }

    // ---- phase 0a: gate sums -------------------------------------------------------------------
    // d = sum of g over tokens 16I+1 .. tok (the lane's decay relative to the block's first
    // token, natural log), a prefix sum across the 16 lanes of a DPP row with the first token's
    // term removed.  The block sums go through LDS to give, per channel, G at each block's
    // first token (G[16I]) and G_last = G at the last valid token.
    // (With the scalar gate every channel of a token has the same gate: one scan per lane.)
    float gv[8 * KBW], d[8 * KBW];
    if constexpr (SG) {
        const float gs = tv ? gsv : 0.f;
        const float ds = row_scan16(n16 == 0 ? 0.f : gs);
#pragma unroll
        for (int i = 0; i < 8 * KBW; ++i) {
            gv[i] = gs;
            d[i] = ds;
        }
    } else {
        if constexpr (GM == 2) {   // g = lower_bound * sigmoid(exp(A_log) (g_raw + dt_bias))
            const float ts = exp2_fast(alog * kLog2e);
#pragma unroll
            for (int i = 0; i < 8 * KBW; ++i) {
                const float x = ts * ((float)xgr[i >> 3][i & 7] + xg[i >> 2][i & 3]);
                // the hardware reciprocal (1 ulp) instead of a correctly rounded division:
                // raw-gate intra at 8K 23.0-23.5 -> 21.6-22.2 us
                gv[i] = p.lower_bound * __builtin_amdgcn_rcpf(1.0f + exp2_fast(-x * kLog2e));
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8 * KBW; ++i) gv[i] = xg[i >> 2][i & 3];
        }
        if (n < kChunk) {   // a tail chunk: rows past it add nothing
#pragma unroll
            for (int i = 0; i < 8 * KBW; ++i) gv[i] = tv ? gv[i] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8 * KBW; ++i) d[i] = row_scan16(n16 == 0 ? 0.f : gv[i]);
    }
    if (n16 == 0 || n16 == 15) {   // block-first gates and block sums, 8 channels per store pair
        float* dst = (n16 == 0 ? sFirst : sDlast) + I * 128 + 8 * q4;
#pragma unroll
        for (int i = 0; i < KBW; ++i) {
            f32x4 a, c;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                a[e] = n16 == 0 ? gv[8 * i + e] : d[8 * i + e];
                c[e] = n16 == 0 ? gv[8 * i + 4 + e] : d[8 * i + 4 + e];
            }
            *reinterpret_cast<f32x4*>(dst + 32 * (kb0 + i)) = a;
            *reinterpret_cast<f32x4*>(dst + 32 * (kb0 + i) + 4) = c;
        }
    }
    __syncthreads();
    if (tid < D) {
        const int c = tid;
        float Gr[4];
        float acc = 0.f;
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            Gr[J] = acc + sFirst[J * 128 + c];
            acc = Gr[J] + sDlast[J * 128 + c];
        }
        const float Gl = acc;
        const int PI[6] = {1, 2, 2, 3, 3, 3};
        const int PJ[6] = {0, 0, 1, 0, 1, 2};
#pragma unroll
        for (int u = 0; u < 6; ++u)
            sVec[(VEC_BV + u) * 128 + c] = exp2_fast((Gr[PI[u]] - Gr[PJ[u]]) * kLog2e);
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            sVec[(VEC_C + J) * 128 + c] = exp2_fast((Gl - Gr[J]) * kLog2e);
            sVecA[J * 128 + c] = exp2_fast(Gr[J] * kLog2e);
        }
        DevStore(p.Gf + size_t(rec) * D, D * 4).put(unsigned(c) * 4, exp2_fast(Gl * kLog2e));
    }

    // ---- phase 1: normalised, decayed operands in registers; K_dec record ---------------------
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int i = 0; i < KBW; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float fq = (float)xq[i][e], fk = (float)xk[i][e];
            sq += fq * fq;
            sk += fk * fk;
        }
    sq += __shfl_xor(sq, 16);
    sq += __shfl_xor(sq, 32);
    sk += __shfl_xor(sk, 16);
    sk += __shfl_xor(sk, 32);
    if constexpr (HV == 2) {   // this half's sums of squares for the other half's wave
        if (q4 == 0) {
            sNrm[(hc * 64 + tok) * 2] = sq;
            sNrm[(hc * 64 + tok) * 2 + 1] = sk;
        }
    }
    __syncthreads();   // vector rows (and the half sums) ready; first/dlast dead
    if constexpr (HV == 2) {
        sq += sNrm[((hc ^ 1) * 64 + tok) * 2];
        sk += sNrm[((hc ^ 1) * 64 + tok) * 2 + 1];
    }
    float qn, kn, bt;
    {
        const bool l2 = (p.flags & KDA_QK_L2NORM) != 0;
        // a zero factor removes the clamped rows past the tail from every q/k product
        // (the hardware reciprocal square root and reciprocal, 1 ulp, for the correctly
        // rounded quotients: no measurable difference in any parity margin)
        // (the query factor carries the output scale, so Aqk and Q~ need no product with it)
        qn = !tv ? 0.f : (l2 ? __builtin_amdgcn_rsqf(sq + 1e-6f) : 1.0f) * p.scale;
        kn = !tv ? 0.f : (l2 ? __builtin_amdgcn_rsqf(sk + 1e-6f) : 1.0f);
        bt = 0.f;
        if (tv)
            bt = (p.flags & KDA_BETA_SIGMOID)
                     ? __builtin_amdgcn_rcpf(1.0f + exp2_fast(-braw * kLog2e))
                     : braw;
    }
    if (q4 == 0 && hc == 0) sBeta[tok] = bt;

    float Lk[8 * KBW], Lq[8 * KBW];
    // the diagonal T and Aqk blocks of row block I (this wave's channels): both sides are this
    // wave's own rows, so they are formed here, beside the operands, with no LDS exchange.  The
    // key side KF = k_j exp(G[16I] - G_j) < 2^109 stays in bf16; masked entries may be huge and
    // are removed by select.  T takes both sides as bf16 hi/lo pairs (three terms; with single
    // bf16 operands the rounding of T was half of the error of a final state without decay),
    // Aqk the hi parts.
    f32x4 aTd = {0.f, 0.f, 0.f, 0.f}, aQd = {0.f, 0.f, 0.f, 0.f};
    {
        const DevStore kdst(p.Kf + size_t(rec) * (64 * D), 64 * D * 2);
        const int s_k = I >> 1;
        const int lane_k = (2 * (I & 1) + (q4 >> 1)) * 16 + n16;
        const int j0 = 4 * (q4 & 1);
#pragma unroll
        for (int i = 0; i < KBW; ++i) {
            const int kb = kb0 + i;
            f16x8 kd;
            float kf[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int ii = 8 * i + e;
                const int c = 32 * kb + 8 * q4 + e;
                // e^{d} <= 1 and e^{-d} < 2^109 (d over at most 15 tokens, g >= -5)
                const float dd = d[ii] * kLog2e;
                const float ef = exp2_fast(dd);
                const float ff = exp2_fast(-dd);
                const float kv = (float)xk[i][e] * kn;
                Lk[ii] = kv * ef;
                Lq[ii] = (float)xq[i][e] * qn * ef;
                kf[e] = kv * ff;
                kd[e] = (_Float16)(kf[e] * sVec[(VEC_C + I) * 128 + c]);   // K_dec <= |k|, one fp16 value
            }
            {
                bf16x8 kh, kl, lh, ll, qh;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    SPLIT_BF16(kf[e], kh[e], kl[e]);
                    SPLIT_BF16(Lk[8 * i + e], lh[e], ll[e]);
                    qh[e] = (__bf16)Lq[8 * i + e];
                }
                aTd = mfma(kh, lh, aTd);
                aTd = mfma(kh, ll, aTd);
                aTd = mfma(kl, lh, aTd);
                aQd = mfma(kh, qh, aQd);
            }
            // the key operand of every later row block I2 > I: k_j exp(G[16 I2] - G_j) <= 1, in
            // fp16 (11 bits; terms below its range are under 2^-24 and dropped)
            for (int I2 = I + 1; I2 < 4; ++I2) {
                const int pi = pair_index(I2, I);
                const float* bv = sVec + (VEC_BV + pi) * 128 + 32 * kb + 8 * q4;
                f16x8 r;
#pragma unroll
                for (int e = 0; e < 8; ++e) r[e] = (_Float16)(kf[e] * bv[e]);
                sR[(pi * KB + kb) * 64 + lane] = r;
            }
            // K_dec^T fragments of Dk tiles 2kb, 2kb+1: [mt D/16][s 2][lane 64][8] fp16
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
                const f16x4 th = to_f16x4(mfma(kd, sel_nat16(hh, q4, n16), zero));
                const int mt = 2 * kb + hh;
                kdst.put(unsigned(((mt * 2 + s_k) * 64 + lane_k) * 8 + j0) * 2, th);
            }
        }
    }
    __syncthreads();   // scaled key blocks, sBeta ready

    // ---- phase 2: T and Aqk blocks of row block I below the diagonal, on MFMA ------------------
    // Both products use the row block's own operands relative to its first token 16I,
    // k_i exp(G_i - G[16I]) <= 1 and q_i exp(G_i - G[16I]); the key side arrives scaled by its
    // owner wave to k_j exp(G[16I] - G_j) <= 1.  Both sides, at most 1 in magnitude, are fp16.
    // With two waves per block each sums over its channel half; the second half's sums pass
    // through LDS (T's after the T blocks, Aqk's in its own not yet written block slots) to the
    // first half's wave, which adds them and stores T and Aqk.
    // The key side is the A operand, so the accumulators hold the transposed blocks: lane
    // (q4, n16) has row i = 16I + n16 and the four consecutive columns 16J + 4q4 .. +3, one
    // 16-byte store per block into the row-major block below.
    f32x4 aT[4], aQ[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) {
        const bool dg = J == I;
        aT[J] = dg ? aTd : f32x4{0.f, 0.f, 0.f, 0.f};
        aQ[J] = dg ? aQd : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (I > 0) {
        f16x8 Lkh16[KBW], Lqh16[KBW];
#pragma unroll
        for (int i = 0; i < KBW; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                Lkh16[i][e] = (_Float16)Lk[8 * i + e];
                Lqh16[i][e] = (_Float16)Lq[8 * i + e];
            }
#pragma unroll
        for (int J = 0; J < 3; ++J) {
            if (J >= I) continue;
#pragma unroll
            for (int i = 0; i < KBW; ++i) {
                const f16x8 bf = sR[(pair_index(I, J) * KB + kb0 + i) * 64 + lane];
                aT[J] = mfma(bf, Lkh16[i], aT[J]);
                aQ[J] = mfma(bf, Lqh16[i], aQ[J]);
            }
        }
    }
    if constexpr (HV == 2) {
        if (hc == 1) {
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                if (J > I) continue;
                *reinterpret_cast<f32x4*>(sTp + blk(I, J) * 256 + 4 * lane) = aT[J];
                *reinterpret_cast<f32x4*>(sAqk + blk(I, J) * BLK_SZ + 4 * lane) = aQ[J];
            }
        }
        __syncthreads();   // the second halves' sums
    }
    // ---- phase 3: Ainv = (I + T)^-1 in fp32 -------------------------------------------------------
    // With D' the block diagonal of I + T (inverses Dinv_I) and L its blocks below the diagonal,
    // I + T = D' (I + N) with N = D'^-1 L, and N^4 = 0 (four block rows), so
    // (I + T)^-1 = (I - N + N^2 - N^3) D'^-1.  The diagonal blocks are inverted by forward
    // substitution (one column per lane, each row's dot product in four partial sums), the rest
    // on the fp32 MFMA as 16 x 16 products:
    //   N_IJ = Dinv_I T_IJ;  Ainv_{J+1,J} = -N_{J+1,J} Dinv_J;
    //   Ainv_20 = M_20 Dinv_0, M_20 = N_21 N_10 - N_20;  Ainv_31 = M_31 Dinv_1, M_31 = N_32 N_21 - N_31;
    //   Ainv_30 = M_30 Dinv_0, M_30 = Z_30 - N_32 M_20, Z_30 = N_31 N_10 - N_30.
    // (Block forward substitution down a block column is a chain of nine such products.)
    // Four waves: the wave that forms row block I of T inverts its diagonal block and forms N_IJ
    // (J < I) in place in the T blocks with no workgroup barrier (its own LDS accesses stay in
    // order); after one barrier every block below the diagonal comes out of one phase, the
    // M_20, M_30 chain (three products deep) in one wave.  Eight waves: the same products in four
    // barrier-separated levels spread over the waves (measured faster there).
    const int lr = lane & 15, lk = lane >> 4;
    auto tb = [&](int I2, int J2) { return sT + blk(I2, J2) * BLK_SZ; };
    auto ab = [&](int I2, int J2) { return sAi + blk(I2, J2) * BLK_SZ; };
    // acc + X Y for 16 x 16 blocks of row stride BLK_LD; lane (lk, lr) holds rows 4 lk + i,
    // column lr of the result
    auto mm = [&](const float* X, const float* Y, f32x4 acc) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[lr * BLK_LD + 4 * ks + lk],
                                                       Y[(4 * ks + lk) * BLK_LD + lr], acc,
                                                       0, 0, 0);
        return acc;
    };
    auto put = [&](float* dst, f32x4 v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(4 * lk + i) * BLK_LD + lr] = v[i];
    };
    auto get = [&](const float* src) {
        f32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = src[(4 * lk + i) * BLK_LD + lr];
        return v;
    };
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    if (hc == 0) {   // T and Aqk blocks of row block I
        const int i = 16 * I + n16;   // this lane's row
        const float bi = sBeta[i];
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            if (J > I) continue;
            float* tbl = tb(I, J);
            float* qb2 = sAqk + blk(I, J) * BLK_SZ;
            if constexpr (HV == 2) {   // (the second half's sums, read before this wave writes)
                aT[J] += *reinterpret_cast<const f32x4*>(sTp + blk(I, J) * 256 + 4 * lane);
                aQ[J] += *reinterpret_cast<const f32x4*>(qb2 + 4 * lane);
            }
            f32x4 t4, q4v;
            if (J < I) {   // below the diagonal block every entry is kept
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    t4[r] = bi * aT[J][r];
                    q4v[r] = aQ[J][r];
                }
            } else {       // the diagonal block: T strictly lower, Aqk lower with the diagonal
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int jj = 16 * J + 4 * q4 + r;
                    t4[r] = (i > jj) ? bi * aT[J][r] : 0.f;
                    q4v[r] = (i >= jj) ? aQ[J][r] : 0.f;
                }
            }
            *reinterpret_cast<f32x4*>(tbl + n16 * BLK_LD + 4 * q4) = t4;
            *reinterpret_cast<f32x4*>(qb2 + n16 * BLK_LD + 4 * q4) = q4v;
        }
        if constexpr (HV == 1) {
            wave_lds_fence();
            if (lane < 16) {   // Dinv_I, column `lane`, over T's diagonal block (row i's
                               // elements are all read before its result is stored)
                float* const db = tb(I, I);
                float x[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float s4[4] = {(r == lane) ? 1.f : 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int m = 0; m < r; ++m) s4[(r - 1 - m) & 3] -= db[r * BLK_LD + m] * x[m];
                    x[r] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) db[r * BLK_LD + lane] = x[r];
            }
            wave_lds_fence();
            f32x4 nb[3];   // N_IJ, J < I, in place of T_IJ (only this wave reads it until the barrier)
#pragma unroll
            for (int J = 0; J < 3; ++J)
                if (J < I) nb[J] = mm(tb(I, I), tb(I, J), zero);
#pragma unroll
            for (int J = 0; J < 3; ++J)
                if (J < I) put(tb(I, J), nb[J]);
        }
    }
    // operands kept for later phases: Q~ = scale * q * exp(G) and K~ hi/lo
    float Qt[8 * KBW];
    bf16x8 bkh[KBW], bkl[KBW];
    auto keep_operands = [&]() {
#pragma unroll
        for (int i = 0; i < KBW; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float a = sVecA[I * 128 + 32 * (kb0 + i) + 8 * q4 + e];
                Qt[8 * i + e] = Lq[8 * i + e] * a;
                SPLIT_BF16(Lk[8 * i + e] * a, bkh[i][e], bkl[i][e]);   // K~ (beta goes with Ainv)
            }
    };
    if constexpr (HV == 2) keep_operands();
    __syncthreads();   // T and Aqk ready (four waves: N below the diagonal, Dinv on it)
    if constexpr (HV == 1) {
        keep_operands();   // independent work beside the product chains
        float* const sM20 = sTmp;
        float* const sM31 = sTmp + BLK_SZ;
        float* const sM30 = sTmp + 2 * BLK_SZ;
        if (w == 0) {   // the M_20, M_30 chain
            const f32x4 m20 = mm(tb(2, 1), tb(1, 0), -get(tb(2, 0)));
            const f32x4 z30 = mm(tb(3, 1), tb(1, 0), -get(tb(3, 0)));
            put(sM20, m20);
            wave_lds_fence();
            put(sM30, -mm(tb(3, 2), sM20, -z30));
            const f32x4 a20 = mm(sM20, tb(0, 0), zero);
            wave_lds_fence();
            const f32x4 a30 = mm(sM30, tb(0, 0), zero);
            put(ab(2, 0), a20);
            put(ab(3, 0), a30);
        } else if (w == 1) {   // the M_31 chain; Dinv_0, Dinv_1 into Ainv
            put(sM31, mm(tb(3, 2), tb(2, 1), -get(tb(3, 1))));
            put(ab(0, 0), get(tb(0, 0)));
            put(ab(1, 1), get(tb(1, 1)));
            wave_lds_fence();
            put(ab(3, 1), mm(sM31, tb(1, 1), zero));
        } else if (w == 2) {   // Ainv_10, Ainv_21; Dinv_2 into Ainv
            const f32x4 a10 = -mm(tb(1, 0), tb(0, 0), zero);
            const f32x4 a21 = -mm(tb(2, 1), tb(1, 1), zero);
            put(ab(1, 0), a10);
            put(ab(2, 1), a21);
            put(ab(2, 2), get(tb(2, 2)));
        } else {   // Ainv_32; Dinv_3 into Ainv
            put(ab(3, 2), -mm(tb(3, 2), tb(2, 2), zero));
            put(ab(3, 3), get(tb(3, 3)));
        }
    } else {
        if (w == 0) {   // all four Dinv in one wave: block lane >> 4, column lane & 15 (the
                        // same substitution, written out at each site: as a shared helper the
                        // compiler's register use grew past the eight-wave form's 128)
            const int g = lane >> 4, col = lane & 15;
            const float* const tw = sT + blk(g, g) * BLK_SZ;
            float* const aw = sAi + blk(g, g) * BLK_SZ;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float s4[4] = {(r == col) ? 1.f : 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int m = 0; m < r; ++m) s4[(r - 1 - m) & 3] -= tw[r * BLK_LD + m] * x[m];
                x[r] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) aw[r * BLK_LD + col] = x[r];
        }
        __syncthreads();
        constexpr int NW = 4 * HV;   // waves of the workgroup
        float* const sM20 = sTmp;
        float* const sM31 = sTmp + BLK_SZ;
        float* const sZ30 = sTmp + 2 * BLK_SZ;   // Z_30, then M_30
        for (int t = w; t < 6; t += NW) {   // level 1, blocks (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
            const int I2 = t < 1 ? 1 : (t < 3 ? 2 : 3);
            const int J2 = t - (I2 * (I2 - 1)) / 2;
            put(tb(I2, J2), mm(ab(I2, I2), tb(I2, J2), zero));
        }
        __syncthreads();
        for (int t = w; t < 6; t += NW) {   // level 2
            if (t < 3)
                put(ab(t + 1, t), -mm(tb(t + 1, t), ab(t, t), zero));
            else if (t == 3)
                put(sM20, mm(tb(2, 1), tb(1, 0), -get(tb(2, 0))));
            else if (t == 4)
                put(sM31, mm(tb(3, 2), tb(2, 1), -get(tb(3, 1))));
            else
                put(sZ30, mm(tb(3, 1), tb(1, 0), -get(tb(3, 0))));
        }
        __syncthreads();
        for (int t = w; t < 3; t += NW) {   // level 3
            if (t == 0)
                put(ab(2, 0), mm(sM20, ab(0, 0), zero));
            else if (t == 1)
                put(ab(3, 1), mm(sM31, ab(1, 1), zero));
            else
                put(sZ30, get(sZ30) - mm(tb(3, 2), sM20, zero));   // read before write, one wave
        }
        __syncthreads();
        if (w == 0) put(ab(3, 0), mm(sZ30, ab(0, 0), zero));   // level 4
    }
    __syncthreads();   // Ainv ready; T and the staging tiles dead

    // ---- phase 3b: token-major tiles of K~ hi/lo (phi channel order) and V ---------------------
    if (!tv) {   // rows past the tail (v was read clamped)
#pragma unroll
        for (int i = 0; i < KBW; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) xv[i][e] = (__bf16)0.f;
    }
    {
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const bf16x8 sp = sel_phi(hh, q4, n16);
            const bf16x8 sn = sel_nat(hh, q4, n16);
#pragma unroll
            for (int i = 0; i < KBW; ++i) {
                const int t = 2 * (kb0 + i) + hh;
                tile_put(sKtH, t, I, q4, n16, to_bf16x4(mfma(bkh[i], sp, zero)));
                tile_put(sKtL, t, I, q4, n16, to_bf16x4(mfma(bkl[i], sp, zero)));
                tile_put(sVt, t, I, q4, n16, to_bf16x4(mfma(xv[i], sn, zero)));
            }
        }
    }
    __syncthreads();

    // ---- phase 4: W^T (phi channel tiles) and U for token block I, three-term hi/lo ----------
    const int nks = (I >= 2) ? 2 : 1;  // 32-token K steps that reach the diagonal
    bf16x4 wT[NTW], uT[NTW];
    {
        f32x4 accW[NTW], accU[NTW];
#pragma unroll
        for (int f = 0; f < NTW; ++f) {
            accW[f] = f32x4{0.f, 0.f, 0.f, 0.f};
            accU[f] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        for (int s = 0; s < nks; ++s) {
            // (Ainv diag beta)[16I + n16][32s + 8q4 + e]: B fragment of
            // W^T = K~^T (Ainv diag beta)^T and A fragment of U = (Ainv diag beta) V, as hi/lo
            float ai[8];
            blk_row8(sAi, I, s, q4, n16, ai);
            bf16x8 ah, al;
#pragma unroll
            for (int e = 0; e < 8; ++e) SPLIT_BF16(ai[e] * sBeta[32 * s + 8 * q4 + e], ah[e], al[e]);
#pragma unroll
            for (int f = 0; f < NTW; ++f) {
                const bf16x8 xh = tile_get(sKtH, tw0 + f, 4 * s + q4, n16);
                const bf16x8 xl = tile_get(sKtL, tw0 + f, 4 * s + q4, n16);
                accW[f] = mfma(xh, ah, accW[f]);
                accW[f] = mfma(xl, ah, accW[f]);
                accW[f] = mfma(xh, al, accW[f]);
            }
            // V is exact in bf16: two terms carry the product to the split's precision
#pragma unroll
            for (int f = 0; f < NTW; ++f) {
                const bf16x8 vv = tile_get(sVt, tw0 + f, 4 * s + q4, n16);
                accU[f] = mfma(ah, vv, accU[f]);
                accU[f] = mfma(al, vv, accU[f]);
            }
        }
        // W^T accumulator: lane (q4, n16) holds W[token 16I + n16][32kb + 8q4 + 4hf + r] for
        // tile 2kb + hf, so the pair of tiles is the W fragment the scan multiplies.
        const DevStore wdst(p.Wf + size_t(rec) * (64 * D), 64 * D * 2);
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < KBW; ++i) {
            bf16x8 oh;   // (bf16 for the transpose below; the record takes fp16)
            f16x8 wh;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                oh[r] = (__bf16)accW[2 * i][r];
                oh[4 + r] = (__bf16)accW[2 * i + 1][r];
                wh[r] = (_Float16)accW[2 * i][r];
                wh[4 + r] = (_Float16)accW[2 * i + 1][r];
            }
            wdst.put(unsigned((I * KB + kb0 + i) * 64 + lane) * 16, wh);
            // token-major -W (phi channel order) for Q' = Q~ + Aqk (-W): a selection with -1
            wT[2 * i] = to_bf16x4(mfma(oh, sel_phi(0, q4, n16, true), zero));
            wT[2 * i + 1] = to_bf16x4(mfma(oh, sel_phi(1, q4, n16, true), zero));
        }
        // U accumulator: lane (q4, n16) holds U[16I + 4q4 + r][16nt + n16]
        const DevStore udst(p.Uf + size_t(rec) * (64 * D), 64 * D * 2);
#pragma unroll
        for (int f = 0; f < NTW; ++f) {
            udst.put(unsigned(((tw0 + f) * 4 + I) * 64 + lane) * 8, to_f16x4(accU[f]));
            uT[f] = to_bf16x4(accU[f]);
        }
    }
    __syncthreads();   // every wave is done with the K~ and V tiles
#pragma unroll
    for (int f = 0; f < NTW; ++f) {
        tile_put(sW, tw0 + f, I, q4, n16, wT[f]);
        tile_put(sU, tw0 + f, I, q4, n16, uT[f]);
    }
    __syncthreads();

    // ---- phase 5: O_intra^T = U^T Aqk^T and Q'^T = Q~^T - W^T Aqk^T (token block I) --------
    {
        f32x4 accO[NTW], accQ[NTW];
#pragma unroll
        for (int f = 0; f < NTW; ++f) {
            accO[f] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int i = f >> 1, hf = f & 1;
#pragma unroll
            for (int r = 0; r < 4; ++r) accQ[f][r] = Qt[i * 8 + 4 * hf + r];
        }
        for (int s = 0; s < nks; ++s) {
            float aq[8];
            blk_row8(sAqk, I, s, q4, n16, aq);
            bf16x8 qh, ql;
#pragma unroll
            for (int e = 0; e < 8; ++e) SPLIT_BF16(aq[e], qh[e], ql[e]);
#pragma unroll
            for (int f = 0; f < NTW; ++f) {
                const bf16x8 a = tile_get(sU, tw0 + f, 4 * s + q4, n16);
                accO[f] = mfma(a, qh, accO[f]);
                accO[f] = mfma(a, ql, accO[f]);
            }
#pragma unroll
            for (int f = 0; f < NTW; ++f) {
                const bf16x8 a = tile_get(sW, tw0 + f, 4 * s + q4, n16);   // -W
                accQ[f] = mfma(a, qh, accQ[f]);
                accQ[f] = mfma(a, ql, accQ[f]);
            }
        }
        const DevStore odst(p.Of + size_t(rec) * (64 * D), 64 * D * 2);
#pragma unroll
        for (int f = 0; f < NTW; ++f)
            odst.put(unsigned(((tw0 + f) * 4 + I) * 64 + lane) * 8, to_bf16x4(accO[f]));
        const DevStore qdst(p.Qf + size_t(rec) * (64 * D), 64 * D * 2);
#pragma unroll
        for (int i = 0; i < KBW; ++i) {
            f16x8 o;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                o[r] = (_Float16)accQ[2 * i][r];
                o[4 + r] = (_Float16)accQ[2 * i + 1][r];
            }
            qdst.put(unsigned((I * KB + kb0 + i) * 64 + lane) * 16, o);
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Inter-chunk scan kernels
// ---------------------------------------------------------------------------------------------
//
// A scan workgroup walks chunks of one (sequence, value head) for NT 16-row Dv tiles.  Each
// step needs the chunk's W, Q' and K_dec (all 64 tokens, all 128 key channels) and gamma,
// which do not depend on the Dv tile, and the tile's U and O_intra fragments.  Each wave loads
// the fragments it multiplies straight into registers, one chunk ahead (two register sets,
// alternated by unrolling the chunk loop by two, so no register copy forces an early wait).
//
// Two-level form for few (sequence, head) chains: a sequence of C chunks is cut into P
// segments.  Chunk c maps the state affinely, S -> S M_c + N_c with M_c = Diag(gamma_c) -
// W_c^T K_dec,c, so segment s has S_out = S_in P_s + N_s, and inside segment s the state
// entering chunk c is S_in P_(..c) + N_(..c) (products and sums over the segment's earlier
// chunks).  kda_seg_kernel walks every segment at once from S = 0 (segment 0 from the initial
// state), writing N_s and the outputs O0_c = Q'_c N_(..c)^T + O_intra,c, and from the identity,
// writing P_s and R_c = Q'_c P_(..c)^T; kda_combine_kernel forms S_in(s) on MFMA, and
// kda_out_kernel completes out_c = O0_c + R_c S_in(s)^T for every chunk of segment s >= 1 at
// once.  The sequential depth is C/P chunk steps plus P - 1 combine steps.

// Head-dim constants of the scan kernels (d_k = d_v = D; four waves split the Dk rows).
template <int D>
struct HD {
    static constexpr int KB = D / 32;    // 32-channel K steps of a product over Dk
    static constexpr int MW = D / 64;    // 16-row Dk tiles per wave
    static constexpr int TILES = D / 16; // 16-row Dv tiles per head
    static constexpr int SLD = D + 8;    // fp16 row stride of the LDS state tile (hi or lo)
};
constexpr int VN_LD = 72;   // fp16 [BV][72]   V_new^T tile (hi or lo), row = value channel

// What a chunk step writes besides the state update.
enum OutMode {
    OUT_FINAL = 1,   // out = Q' S^T + O_intra in bf16, valid tokens only
    OUT_O0 = 2,      // O0 = Q' S^T + O_intra in bf16, workspace (state from a zero start)
    OUT_R = 3,       // R = Q' S^T in bf16, workspace (state rows of the transfer matrix)
};

template <int NT, int D>
struct ChunkFrags {
    f16x8 w[HD<D>::KB];                           // W (fp16), token tile w, 32-channel block kb
    f16x8 qp[HD<D>::KB];                          // Q' (fp16), token tile w
    f16x8 kh[HD<D>::MW][2];                       // K_dec^T (fp16), Dk tile MW*w+mt, token step s
    float gm[HD<D>::MW];                          // gamma_last, Dk row 4 q4 + (lane & 3) of
                                                  // tile MW*w+mt (quad-broadcast at use), or
    float g[D / 64];                              // gamma_last[lane D/64 ..] (wave 0, GLDS)
    f16x4 u[NT];                                  // U (fp16), token tile w, Dv tile
    bf16x4 o[NT];                                 // O_intra (bf16), token tile w, Dv tile
};

// PART 1: the operands of a step's first products (W, Q', U, O_intra); PART 2: those of its
// state update (K_dec, gamma); PART 0: all.
// GLDS: wave 0 loads gamma for the workgroup (one load instead of one per wave and Dk tile) and
// the step passes it on through LDS.  Taken by the four-wave one-tile scan with the record
// prefetch wave (at head dim 64; at 128 that scan now runs the eight-wave walk), measured on the
// 128K workload when it ran this walk: 2.54 -> 2.31 ms; slower for the segment pass.  With GLDS
// every operand is also a buffer load (ld_op): the compiler then keeps no per-chunk address
// registers that alias loaded data, and the chunk loop loses the full drain of outstanding
// loads it had at its top (128K scan 2.24 -> 1.98 ms; no faster for the other scans).
template <int NT, int D, int PART = 0, bool GLDS = false>
__device__ __forceinline__ void load_chunk(const Params& p, int64_t rec, int w, int lane,
                                           int dv_tile0, ChunkFrags<NT, D>& f) {
    constexpr int KB = HD<D>::KB, MW = HD<D>::MW;
    if constexpr (PART != 2) {
        constexpr unsigned RB = 64 * D * 2;   // bytes of one record array
        const _Float16* wsrc = p.Wf + size_t(rec) * (64 * D);
        const _Float16* qsrc = p.Qf + size_t(rec) * (64 * D);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            f.w[kb] = ld_op<GLDS, f16x8>(wsrc, RB, unsigned((w * KB + kb) * 64 + lane) * 16);
            f.qp[kb] = ld_op<GLDS, f16x8>(qsrc, RB, unsigned((w * KB + kb) * 64 + lane) * 16);
        }
        const _Float16* usrc = p.Uf + size_t(rec) * (64 * D);
        const __bf16* osrc = p.Of + size_t(rec) * (64 * D);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int dt = dv_tile0 + nt;
            f.u[nt] = ld_op<GLDS, f16x4>(usrc, RB, unsigned((dt * 4 + w) * 64 + lane) * 8);
            f.o[nt] = ld_op<GLDS, bf16x4>(osrc, RB, unsigned((dt * 4 + w) * 64 + lane) * 8);
        }
    }
    if constexpr (PART != 1) {
        const _Float16* ksrc = p.Kf + size_t(rec) * (64 * D);
#pragma unroll
        for (int mt = 0; mt < MW; ++mt)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int off = (((MW * w + mt) * 2 + s) * 64 + lane) * 8;
                f.kh[mt][s] = ld_op<GLDS, f16x8>(ksrc, 64 * D * 2, unsigned(off) * 2);
            }
        if constexpr (GLDS) {
            if (w == 0) {
                const float* gsrc = p.Gf + size_t(rec) * D;
                if constexpr (D == 128) {
                    const float2 x = ld_op<GLDS, float2>(gsrc, D * 4, unsigned(lane) * 8);
                    f.g[0] = x.x;
                    f.g[D / 64 - 1] = x.y;
                } else {
                    f.g[0] = ld_op<GLDS, float>(gsrc, D * 4, unsigned(lane) * 4);
                }
            }
        } else {
            const float* gsrc = p.Gf + size_t(rec) * D;
#pragma unroll
            for (int mt = 0; mt < MW; ++mt)
                f.gm[mt] = ld_op<GLDS, float>(
                    gsrc, D * 4, unsigned(16 * (MW * w + mt) + 4 * (lane >> 4) + (lane & 3)) * 4);
        }
    }
}

// The four values of a lane quad, each broadcast to every lane of the quad (DPP quad_perm
// [r,r,r,r]): with lane 4k + r holding row 4 q4 + r of a 16-row tile, every lane gets the four
// rows 4 q4 .. 4 q4 + 3 of its accumulator fragment.  Each lane then loads one dword of
// gamma_last per Dk tile instead of a 16-byte vector that all 16 lanes of its row share.
__device__ __forceinline__ f32x4 quad_bcast(float x) {
    const int v = __builtin_bit_cast(int, x);
#define KDA_QUAD(c) __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, c, 0xf, 0xf, false))
    const f32x4 r = {KDA_QUAD(0x00), KDA_QUAD(0x55), KDA_QUAD(0xaa), KDA_QUAD(0xff)};
#undef KDA_QUAD
    return r;
}

// Writes one fp32 state fragment (4 consecutive Dk values of one Dv row) as an fp16 hi/lo pair,
// the operands of the combine's fp16 products (about 22 significant bits; the state's magnitude
// is bounded by fp16's 65504).
template <int D>
__device__ __forceinline__ void put_state16(_Float16* sSh, _Float16* sSl, int row, int col, f32x4 x) {
    f16x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = (_Float16)x[i];
        l[i] = (_Float16)(x[i] - (float)h[i]);
    }
    *reinterpret_cast<f16x4*>(sSh + row * HD<D>::SLD + col) = h;
    *reinterpret_cast<f16x4*>(sSl + row * HD<D>::SLD + col) = l;
}

// The walks' copy of the state fragment: fp16 (11 significant bits) as the operand of their
// products with W and Q' (fp16 themselves); the state stays fp32 in registers.
template <int D>
__device__ __forceinline__ void put_state_hi(_Float16* sSh, int row, int col, f32x4 x) {
    f16x4 h;
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = (_Float16)x[i];
    *reinterpret_cast<f16x4*>(sSh + row * HD<D>::SLD + col) = h;
}

struct ScanLds {
    _Float16* sh;   // the state, fp16 (the combine: hi/lo)
    _Float16* sl;
    _Float16* vh;   // V_new, fp16 hi/lo
    _Float16* vl;
    float* g;   // gamma_last of the current chunk [D]
};

// One chunk of the scan for this workgroup's Dv tile(s):
//   X = W S^T and (with outputs) Y^T = S Q'^T for token tile w; V_new = U - X (U = 0 for the
//   transfer-matrix pass); out = Y + O_intra (or R = Y); S^T <- gamma * S^T + K_dec^T V_new
//   for this wave's D/4 Dk rows.  `rec` is the chunk's record (workspace outputs).
//   With SPLIT the next chunk's operands (record rec_nxt) load into `nxt` here, in two parts,
//   each issued after the products it must not delay (a wave that issues a burst of loads
//   waits at issue while the compute unit's address unit takes them); without it the caller
//   has issued them all before the step.  Which is faster depends on the kernel (measured).
template <int NT, int D, bool SPLIT, bool GLDS>
__device__ __forceinline__ void scan_step(const Params& p, const ChunkFrags<NT, D>& cur,
                                          ChunkFrags<NT, D>& nxt, int64_t rec_nxt,
                                          f32x4 (&S)[HD<D>::MW][NT], const ScanLds& L, int jc,
                                          int len, size_t ob, size_t os, int dv_tile0) {
    constexpr int KB = HD<D>::KB, MW = HD<D>::MW, SLD = HD<D>::SLD;
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int q4 = lane >> 4;
    const int n16 = lane & 15;

    // X = W S^T (tokens of tile w x Dv); Y^T = S Q'^T (Dv x tokens), S as its fp16 copy
    f32x4 accX[NT], accY[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        accX[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        accY[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int off = (16 * nt + n16) * SLD + 32 * kb + 8 * q4;
            const f16x8 sh = *reinterpret_cast<const f16x8*>(L.sh + off);
            accX[nt] = mfma(cur.w[kb], sh, accX[nt]);
            accY[nt] = mfma(sh, cur.qp[kb], accY[nt]);
        }
    }
    if constexpr (SPLIT) {
        __builtin_amdgcn_sched_barrier(0);
        load_chunk<NT, D, 1>(p, rec_nxt, w, lane, dv_tile0, nxt);
        __builtin_amdgcn_sched_barrier(0);
    }
    const int tok = jc * kChunk + 16 * w + n16;  // output token of this lane
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        f16x4 vh, vl;   // V_new as an fp16 pair, the operand of the fp16 update product
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float x = (float)cur.u[nt][r] - accX[nt][r];
            vh[r] = (_Float16)x;
            vl[r] = (_Float16)(x - (float)vh[r]);
        }
        const int off = (16 * nt + n16) * VN_LD + 16 * w + 4 * q4;
        *reinterpret_cast<f16x4*>(L.vh + off) = vh;
        *reinterpret_cast<f16x4*>(L.vl + off) = vl;
        if (tok < len) {
            bf16x4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = (__bf16)(accY[nt][r] + (float)cur.o[nt][r]);
            *reinterpret_cast<bf16x4*>(p.out + ob + size_t(tok) * os + 16 * (dv_tile0 + nt) +
                                       4 * q4) = o;
        }
    }
    static_assert(!(GLDS && SPLIT), "gamma through LDS comes with unsplit loads");
    if constexpr (GLDS) {
        if (w == 0) {
#pragma unroll
            for (int e = 0; e < D / 64; ++e) L.g[lane * (D / 64) + e] = cur.g[e];
        }
    }
    lds_barrier();

    // S^T <- gamma * S^T + K_dec^T V_new  (Dk rows of this wave x Dv) on the fp16 MFMA: K_dec
    // (one fp16 value, at most |k|) times V_new as an fp16 hi/lo pair
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        f16x8 vh[2], vl[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int off = (16 * nt + n16) * VN_LD + 32 * s + 8 * q4;
            vh[s] = *reinterpret_cast<const f16x8*>(L.vh + off);
            vl[s] = *reinterpret_cast<const f16x8*>(L.vl + off);
        }
#pragma unroll
        for (int mt = 0; mt < MW; ++mt) {
            f32x4 acc = S[mt][nt] * (GLDS ? *reinterpret_cast<const f32x4*>(
                                                L.g + 16 * (MW * w + mt) + 4 * q4)
                                          : quad_bcast(cur.gm[mt]));
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                acc = mfma(cur.kh[mt][s], vh[s], acc);
                acc = mfma(cur.kh[mt][s], vl[s], acc);
            }
            S[mt][nt] = acc;
            put_state_hi<D>(L.sh, 16 * nt + n16, 16 * (MW * w + mt) + 4 * q4, acc);
        }
    }
    if constexpr (SPLIT) {
        __builtin_amdgcn_sched_barrier(0);
        load_chunk<NT, D, 2>(p, rec_nxt, w, lane, dv_tile0, nxt);
    }
    lds_barrier();
}

// Chunks [cb, ce) of one sequence (records rec0 + c * n_v), state in S and in LDS on entry:
// the one-level scan's four-wave walk (its outputs stored plainly; at device scope, as the
// segment pass stores them, the one-level scan's output stream measured slower).
// The prefetch is issued on every step, past the end as a reload of the last chunk (a valid
// record, never used): with the same number of loads in flight on every path, the compiler's
// wait counts let each step wait only for its own operands, not for the next chunk's.
template <int NT, int D, bool SPLIT, bool GLDS = false>
__device__ __forceinline__ void run_chunks(const Params& p, f32x4 (&S)[HD<D>::MW][NT],
                                           const ScanLds& L,
                                           int64_t rec0, int cb, int ce, int len, size_t ob,
                                           size_t os, int dv_tile0) {
    if (cb >= ce) return;
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int last = ce - 1;
    ChunkFrags<NT, D> fa, fb;
    load_chunk<NT, D, 0, GLDS>(p, rec0 + int64_t(cb) * p.n_v, w, lane, dv_tile0, fa);
    for (int jc = cb; jc < ce; jc += 2) {
        const int c1 = jc + 1 < last ? jc + 1 : last;
        if constexpr (!SPLIT)
            load_chunk<NT, D, 0, GLDS>(p, rec0 + int64_t(c1) * p.n_v, w, lane, dv_tile0, fb);
        scan_step<NT, D, SPLIT, GLDS>(p, fa, fb, rec0 + int64_t(c1) * p.n_v, S, L, jc, len, ob,
                                      os, dv_tile0);
        if (jc + 1 >= ce) break;
        const int c2 = jc + 2 < last ? jc + 2 : last;
        if constexpr (!SPLIT)
            load_chunk<NT, D, 0, GLDS>(p, rec0 + int64_t(c2) * p.n_v, w, lane, dv_tile0, fa);
        scan_step<NT, D, SPLIT, GLDS>(p, fb, fa, rec0 + int64_t(c2) * p.n_v, S, L, jc + 1, len,
                                      ob, os, dv_tile0);
    }
}

// Eight-wave chunk step (the segment pass, one 16-row Dv tile; and at head dim 128 the one-level
// scans with the prefetch wave, NT = 1 or 2 Dv tiles).  With four waves every SIMD holds one
// wave of the walk, and nothing covers its LDS and memory waits.  Here waves 0..3 take token
// tile w & 3 of X = W S^T and its V_new, waves 4..7 the same token tile of Y^T = S Q'^T and its
// outputs, for each of the NT Dv tiles, and in the state update each wave takes one 16-row Dk
// tile of every Dv tile (at head dim 64, whose state has four, the X waves alone): the
// workgroup loads exactly what the four-wave step loads (each operand once; W, Q', K_dec and
// gamma once for all NT tiles), with two waves on every SIMD.  Measured at the 8K prefill:
// segment pass 24.5-24.9 -> 23.3-24.0 us.
template <int D, int NT = 1>
struct Frags8 {
    f16x8 a[HD<D>::KB];    // W (X waves) or Q' (Y waves), fp16, token tile w & 3
    f16x8 kh[2];           // K_dec^T of Dk tile w, token steps 0 and 1
    float gm;              // gamma_last of row 4 q4 + (lane & 3) of Dk tile w (quad-broadcast)
    f16x4 u[NT];           // U (X waves), token tile w & 3, Dv tile nt
    bf16x4 o[NT];          // O_intra (Y waves), the same
};

// Every operand of one chunk for a wave of the eight-wave walk: W (X waves) or Q' (Y waves) of
// its token tile, U (X) or O_intra (Y) of that tile and each Dv tile, and the K_dec and gamma
// of its Dk tile.
template <int ROLE, bool WITH_U, int OUT, int D, bool BUF, int NT = 1>
__device__ __forceinline__ void load_chunk8(const Params& p, int64_t rec, int w, int lane,
                                            int dv_tile, Frags8<D, NT>& f) {
    constexpr int KB = HD<D>::KB;
    const int tt = w & 3;
    const size_t rb = size_t(rec) * (64 * D);
    constexpr unsigned RB = 64 * D * 2;
    const _Float16* src = (ROLE == 0 ? p.Wf : p.Qf) + rb;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
        f.a[kb] = ld_op<BUF, f16x8>(src, RB, unsigned((tt * KB + kb) * 64 + lane) * 16);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int uo = (((dv_tile + nt) * 4 + tt) * 64 + lane) * 4;
        if constexpr (ROLE == 0 && WITH_U)
            f.u[nt] = ld_op<BUF, f16x4>(p.Uf + rb, RB, unsigned(uo) * 2);
        if constexpr (ROLE == 1 && (OUT == OUT_FINAL || OUT == OUT_O0))
            f.o[nt] = ld_op<BUF, bf16x4>(p.Of + rb, RB, unsigned(uo) * 2);
    }
    if constexpr (D == 128 || ROLE == 0) {   // the waves that update a Dk tile of the state
#pragma unroll
        for (int s = 0; s < 2; ++s)
            f.kh[s] = ld_op<BUF, f16x8>(p.Kf + rb, RB, unsigned((w * 2 + s) * 64 + lane) * 16);
        f.gm = ld_op<BUF, float>(p.Gf + size_t(rec) * D, D * 4,
                                 unsigned(16 * w + 4 * (lane >> 4) + (lane & 3)) * 4);
    }
}

// One chunk for the workgroup's NT Dv tiles with eight waves (see Frags8); ROLE 0 is an X wave
// (waves 0..3), ROLE 1 a Y wave (4..7), each running its own branch-free copy of the walk.
// Outputs are stored at device scope (the segment pass) or plainly (ONE_LEVEL).
template <int ROLE, bool WITH_U, int OUT, int D, bool ONE_LEVEL = false, int NT = 1>
__device__ __forceinline__ void scan_step8(const Params& p, const Frags8<D, NT>& cur,
                                           f32x4 (&S)[NT], const ScanLds& L, int w, int jc,
                                           int len, size_t ob, size_t os, int dv_tile,
                                           int64_t rec) {
    constexpr int KB = HD<D>::KB, SLD = HD<D>::SLD;
    static_assert(D / 16 == 8 || D / 16 == 4, "one 16-row Dk tile per wave or per X wave");
    const int lane = threadIdx.x & 63;
    const int q4 = lane >> 4;
    const int n16 = lane & 15;
    const int tt = w & 3;

#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        // X = W S^T, or Y^T = S Q'^T, token tile tt, Dv tile nt (S as its fp16 copy)
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int off = (16 * nt + n16) * SLD + 32 * kb + 8 * q4;
            const f16x8 sh = *reinterpret_cast<const f16x8*>(L.sh + off);
            if constexpr (ROLE == 0)
                acc = mfma(cur.a[kb], sh, acc);
            else
                acc = mfma(sh, cur.a[kb], acc);
        }
        const int dt = dv_tile + nt;
        if constexpr (ROLE == 0) {   // V_new as an fp16 pair, the operand of the fp16 update
            f16x4 vh, vl;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = (WITH_U ? (float)cur.u[nt][r] : 0.f) - acc[r];
                vh[r] = (_Float16)x;
                vl[r] = (_Float16)(x - (float)vh[r]);
            }
            const int off = (16 * nt + n16) * VN_LD + 16 * tt + 4 * q4;
            *reinterpret_cast<f16x4*>(L.vh + off) = vh;
            *reinterpret_cast<f16x4*>(L.vl + off) = vl;
        } else {
            const int tok = jc * kChunk + 16 * tt + n16;   // output token of this lane
            bf16x4 yb;
            if constexpr (OUT == OUT_FINAL) {
                if (tok < len) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) yb[r] = (__bf16)(acc[r] + (float)cur.o[nt][r]);
                    if constexpr (!ONE_LEVEL) {
                        const DevStore dst(p.out + ob + size_t(jc) * kChunk * os,
                                           unsigned(kChunk * os * 2));
                        dst.put(unsigned((tok - jc * kChunk) * os + 16 * dt + 4 * q4) * 2, yb);
                    } else {
                        *reinterpret_cast<bf16x4*>(p.out + ob + size_t(tok) * os + 16 * dt +
                                                   4 * q4) = yb;
                    }
                }
            } else if constexpr (OUT == OUT_O0) {
#pragma unroll
                for (int r = 0; r < 4; ++r) yb[r] = (__bf16)(acc[r] + (float)cur.o[nt][r]);
                DevStore(p.O0 + size_t(rec) * (64 * D), 64 * D * 2)
                    .put(unsigned((dt * 4 + tt) * 64 + lane) * 8, yb);
            } else if constexpr (OUT == OUT_R) {   // R in the completion pass's B-operand order
#pragma unroll
                for (int r = 0; r < 4; ++r) yb[r] = (__bf16)acc[r];
                const int lb = (2 * (dt & 1) + (q4 >> 1)) * 16 + n16;
                DevStore(p.Rf + size_t(rec) * (64 * D), 64 * D * 2)
                    .put(unsigned(((tt * KB + (dt >> 1)) * 64 + lb) * 8 + 4 * (q4 & 1)) * 2, yb);
            }
        }
    }
    lds_barrier();

    // S^T <- gamma * S^T + K_dec^T V_new for Dk tile w of each Dv tile, on the fp16 MFMA (at head
    // dim 64, four Dk tiles: the X waves only)
    if constexpr (D == 128 || ROLE == 0) {
        const f32x4 gq = quad_bcast(cur.gm);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f16x8 vh[2], vl[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int off = (16 * nt + n16) * VN_LD + 32 * s + 8 * q4;
                vh[s] = *reinterpret_cast<const f16x8*>(L.vh + off);
                vl[s] = *reinterpret_cast<const f16x8*>(L.vl + off);
            }
            f32x4 a = S[nt] * gq;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                a = mfma(cur.kh[s], vh[s], a);
                a = mfma(cur.kh[s], vl[s], a);
            }
            S[nt] = a;
            put_state_hi<D>(L.sh + 16 * nt * SLD, n16, 16 * w + 4 * q4, a);
        }
    }
    lds_barrier();
}

// Chunks [cb, ce) with the eight-wave step (as run_chunks, state in S and in LDS on entry);
// waves 0..3 run the X copy and waves 4..7 the Y copy of the walk, with the same barriers.
// ONE_LEVEL: the one-level scan (outputs stored plainly, operands as buffer loads); otherwise
// the segment pass (outputs at device scope, plain operand loads): each measured faster there.
template <int ROLE, bool WITH_U, int OUT, int D, bool ONE_LEVEL = false, int NT = 1>
__device__ __forceinline__ void run_walk8(const Params& p, f32x4 (&S)[NT], const ScanLds& L,
                                          int w, int64_t rec0, int cb, int ce, int len,
                                          size_t ob, size_t os, int dv_tile) {
    const int lane = threadIdx.x & 63;
    const int last = ce - 1;
    // the next chunk's loads are written ahead of the step; the compiler issues them after the
    // step's first products, into the registers those products have consumed (the step's own
    // operands arrived during the previous step).  Measured: faster than the loads pinned
    // ahead of the products by a scheduling barrier (segment pass at 8K 22.9 -> 24.0 us), as
    // fast as issuing them two chunks ahead from a third operand set, and faster than loads
    // split around the products (with which the compiler folded the two-step loop into one and
    // drained every load, K_dec's included, at the top of each step)
    Frags8<D, NT> fa, fb;
    load_chunk8<ROLE, WITH_U, OUT, D, ONE_LEVEL, NT>(p, rec0 + int64_t(cb) * p.n_v, w, lane,
                                                     dv_tile, fa);
    for (int jc = cb; jc < ce; jc += 2) {
        const int c1 = jc + 1 < last ? jc + 1 : last;
        load_chunk8<ROLE, WITH_U, OUT, D, ONE_LEVEL, NT>(p, rec0 + int64_t(c1) * p.n_v, w, lane,
                                                         dv_tile, fb);
        scan_step8<ROLE, WITH_U, OUT, D, ONE_LEVEL, NT>(p, fa, S, L, w, jc, len, ob, os,
                                                        dv_tile, rec0 + int64_t(jc) * p.n_v);
        if (jc + 1 >= ce) break;
        const int c2 = jc + 2 < last ? jc + 2 : last;
        load_chunk8<ROLE, WITH_U, OUT, D, ONE_LEVEL, NT>(p, rec0 + int64_t(c2) * p.n_v, w, lane,
                                                         dv_tile, fa);
        scan_step8<ROLE, WITH_U, OUT, D, ONE_LEVEL, NT>(p, fb, S, L, w, jc + 1, len, ob, os,
                                                        dv_tile, rec0 + int64_t(jc + 1) * p.n_v);
    }
}

template <bool WITH_U, int OUT, int D, bool ONE_LEVEL = false, int NT = 1>
__device__ __forceinline__ void run_chunks8(const Params& p, f32x4 (&S)[NT], const ScanLds& L,
                                            int64_t rec0, int cb, int ce, int len, size_t ob,
                                            size_t os, int dv_tile) {
    if (cb >= ce) return;
    const int w = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
    if (w < 4)
        run_walk8<0, WITH_U, OUT, D, ONE_LEVEL, NT>(p, S, L, w, rec0, cb, ce, len, ob, os,
                                                    dv_tile);
    else
        run_walk8<1, WITH_U, OUT, D, ONE_LEVEL, NT>(p, S, L, w, rec0, cb, ce, len, ob, os,
                                                    dv_tile);
}

// Sequences of different lengths (cu_seqlens given) are walked longest first: workgroup rank r
// takes the sequence of rank r in the order of decreasing valid length (ties by index), so the
// long walks start first and the short ones fill the end of the grid (longest processing time
// first).  Every workgroup ranks the lengths itself, from LDS; with more than kRankMax sequences
// the order stays the index order.  Uniform for the workgroup (all its threads call it).
constexpr int kRankMax = 256;
__device__ __forceinline__ int seq_by_rank(const Params& p, int r) {
    if (!p.cu || p.batch <= 1 || p.batch > kRankMax) return r;
    __shared__ int sLen[kRankMax];
    __shared__ int sSeq;
    for (int t = threadIdx.x; t < p.batch; t += blockDim.x) {
        int c0, len, slot0;
        seq_info(p, t, c0, len, slot0);
        sLen[t] = len;
    }
    __syncthreads();
    for (int t = threadIdx.x; t < p.batch; t += blockDim.x) {
        const int lt = sLen[t];
        int rank = 0;
        for (int u = 0; u < p.batch; ++u) {
            const int lu = sLen[u];
            rank += (lu > lt || (lu == lt && u < t)) ? 1 : 0;
        }
        if (rank == r) sSeq = t;
    }
    __syncthreads();
    return sSeq;
}

// Chunk range [cb, ce) of segment `seg` of a sequence with `nchunks` chunks cut into seg_p
// segments of ceil(nchunks / seg_p) chunks.
__device__ __forceinline__ void segment_range(int nchunks, int seg_p, int seg, int& cb, int& ce) {
    const int L = (nchunks + seg_p - 1) / seg_p;
    cb = seg * L;
    ce = cb + L < nchunks ? cb + L : nchunks;
    if (cb > nchunks) cb = nchunks;
}

// Operands of one combine step S <- S P_s + N_s for this wave's Dk tiles M = MW w + mt: the
// A fragments of P_s^T (fp16) and the accumulator fragments of this workgroup's N_s tiles.
template <int NT, int D>
struct CombFrags {
    f16x8 ph[HD<D>::MW][HD<D>::KB];    // P_s[32kb+8q4 .. +7][16M+n16]
    f32x4 n[NT][HD<D>::MW];            // N_s[16(dv_tile0+nt)+n16][16M+4q4 .. +3]
};

template <int NT, int D>
__device__ __forceinline__ void load_comb(const _Float16* Pt, const float* Nst, int dv_tile0,
                                          CombFrags<NT, D>& f) {
    constexpr int KB = HD<D>::KB, MW = HD<D>::MW;
    constexpr int TILES = HD<D>::TILES;
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            f.ph[mt][kb] = *reinterpret_cast<const f16x8*>(
                Pt + (((MW * w + mt) * KB + kb) * 64 + lane) * 8);
        }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MW; ++mt)
            f.n[nt][mt] = *reinterpret_cast<const f32x4*>(
                Nst + (((dv_tile0 + nt) * TILES + MW * w + mt) * 64 + lane) * 4);
}

// S^T <- P_s^T S^T + N_s^T for this wave's Dk rows, i.e. S <- S P_s + N_s, with the state in S
// (registers) and in LDS as an fp16 hi/lo pair (B operand), P_s in fp16: two products on the
// fp16 MFMA.
template <int NT, int D>
__device__ __forceinline__ void combine_step(const CombFrags<NT, D>& f,
                                             f32x4 (&S)[HD<D>::MW][NT], const ScanLds& L) {
    constexpr int KB = HD<D>::KB, MW = HD<D>::MW, SLD = HD<D>::SLD;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int q4 = lane >> 4;
    const int n16 = lane & 15;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int mt = 0; mt < MW; ++mt) {
            f32x4 acc = f.n[nt][mt];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int off = (16 * nt + n16) * SLD + 32 * kb + 8 * q4;
                const f16x8 sh = *reinterpret_cast<const f16x8*>(L.sh + off);
                const f16x8 sl = *reinterpret_cast<const f16x8*>(L.sl + off);
                acc = mfma(f.ph[mt][kb], sh, acc);
                acc = mfma(f.ph[mt][kb], sl, acc);
            }
            S[mt][nt] = acc;
        }
    }
    lds_barrier();   // every wave has read the old state
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int mt = 0; mt < MW; ++mt)
            put_state16<D>(L.sh, L.sl, 16 * nt + n16, 16 * (MW * w + mt) + 4 * q4, S[mt][nt]);
    lds_barrier();
}

// ---------------------------------------------------------------------------------------------
// Record prefetch wave
// ---------------------------------------------------------------------------------------------
//
// The Dv-tile workgroups of one walk all read the same W, Q', K_dec and gamma of each chunk, on
// one XCD.  Walking in step, they all miss in L2 on the same lines at once, and each compute
// unit then streams records from HBM at about half the rate it reaches from L2.  One-level
// scan workgroups that run one per compute unit therefore carry a fifth wave that touches one
// dword of each of its share of a record's lines kPfDist chunks ahead (the shared lines split
// among the walk's workgroups, plus its own U and O_intra tiles), so that the compute waves
// find them in L2.  It keeps in step through the same workgroup barriers as the compute waves
// (two per chunk) and consumes each value four chunks later, so it never waits for a line.
// (Measured on the 128K, 32-head call: 2.99 ms -> 2.49 ms for the scan at a distance of two
// chunks; 3.06 ms at one, 2.47 at three, 2.60 at four.  The segment pass of the two-level
// scan, whose records come from the last-level cache, gains nothing from it.)
constexpr int kPfThreads = kThreads + 64;
constexpr int kPfDist = 2;
constexpr int kPfSlots = 4;   // lines per lane and chunk

template <int D>
struct RecPrefetch {
    const unsigned char* base[kPfSlots];
    unsigned stride[kPfSlots];   // bytes per record of the slot's array
    unsigned ring[4][kPfSlots];
    unsigned sink;

    // Share `part` of `parts` of the shared lines, and the U/O_intra lines of Dv tiles
    // dv_tile0 .. dv_tile0 + own_tiles - 1.
    __device__ __forceinline__ void init(const Params& p, int part, int parts, int dv_tile0,
                                         int own_tiles) {
        constexpr int WL = 64 * D * 2 / 128;   // lines of W, and of Q'
        constexpr int KL = WL;                // K_dec (fp16)
        constexpr int GL = D * 4 / 128;       // gamma
        constexpr int NS = 2 * WL + KL + GL;
        const int sh = (NS + parts - 1) / parts;
        const int s0 = part * sh;
        const int scnt = NS - s0 < sh ? NS - s0 : sh;
        const int ucnt = 16 * own_tiles;      // 2 KiB of U per tile
        const int total = scnt + ucnt + 16 * own_tiles;
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int k = 0; k < kPfSlots; ++k) {
            int li = lane + 64 * k;
            li = li < total ? li : total - 1;
            const unsigned char* b;
            unsigned st;
            size_t off;
            if (li < scnt) {
                const int s = s0 + li;
                if (s < WL) {
                    b = reinterpret_cast<const unsigned char*>(p.Wf); st = 64 * D * 2; off = size_t(s) * 128;
                } else if (s < 2 * WL) {
                    b = reinterpret_cast<const unsigned char*>(p.Qf); st = 64 * D * 2; off = size_t(s - WL) * 128;
                } else if (s < 2 * WL + KL) {
                    b = reinterpret_cast<const unsigned char*>(p.Kf); st = 64 * D * 2; off = size_t(s - 2 * WL) * 128;
                } else {
                    b = reinterpret_cast<const unsigned char*>(p.Gf); st = D * 4; off = size_t(s - 2 * WL - KL) * 128;
                }
            } else if (li < scnt + ucnt) {
                b = reinterpret_cast<const unsigned char*>(p.Uf); st = 64 * D * 2;
                off = size_t(dv_tile0) * 2048 + size_t(li - scnt) * 128;
            } else {
                b = reinterpret_cast<const unsigned char*>(p.Of); st = 64 * D * 2;
                off = size_t(dv_tile0) * 2048 + size_t(li - scnt - ucnt) * 128;
            }
            base[k] = b + off;
            stride[k] = st;
#pragma unroll
            for (int u = 0; u < 4; ++u) ring[u][k] = 0u;
        }
        sink = 0u;
    }

    template <int U>
    __device__ __forceinline__ void touch(int64_t rec) {
#pragma unroll
        for (int k = 0; k < kPfSlots; ++k) {
            sink ^= ring[U][k];
            ring[U][k] = *reinterpret_cast<const unsigned*>(base[k] + size_t(rec) * stride[k]);
        }
    }

    // Keeps the loads alive: the store below never runs (seq_len >= 1 on every launch).
    __device__ __forceinline__ void finish(const Params& p) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int k = 0; k < kPfSlots; ++k) sink ^= ring[u][k];
        if (sink == 0x9e3779b9u && p.seq_len < 0) p.out[threadIdx.x & 63] = (__bf16)0.f;
    }
};

// The prefetch wave's side of a walk over chunks [cb, ce) of records rec0 + c * n_v: chunk c
// + kPfDist is touched while the compute waves work on chunk c, and each chunk passes the two
// barriers of a chunk step (run_chunks: ce - cb steps of scan_step, two barriers each).
template <int D>
__device__ __forceinline__ void prefetch_walk(RecPrefetch<D>& pf, int64_t rec0, int n_v, int cb,
                                              int ce) {
    if (cb >= ce) return;
    const int last = ce - 1;
    auto rec = [&](int c) { return rec0 + int64_t(c < last ? c : last) * n_v; };
    for (int jc = cb; jc < ce; jc += 4) {
        pf.template touch<0>(rec(jc + kPfDist));
        lds_barrier();
        lds_barrier();
        if (jc + 1 >= ce) break;
        pf.template touch<1>(rec(jc + 1 + kPfDist));
        lds_barrier();
        lds_barrier();
        if (jc + 2 >= ce) break;
        pf.template touch<2>(rec(jc + 2 + kPfDist));
        lds_barrier();
        lds_barrier();
        if (jc + 3 >= ce) break;
        pf.template touch<3>(rec(jc + 3 + kPfDist));
        lds_barrier();
        lds_barrier();
    }
}

// Rows past a batch row's valid length (BNSD/BSND with cu_seqlens) are written as zeros, for
// output columns [col0, col0 + ncols) (ncols a multiple of 4).
__device__ __forceinline__ void zero_rows_past_len(const Params& p, int len, size_t ob, size_t os,
                                                   int col0, int ncols) {
    if (p.layout == KDA_LAYOUT_TND || len >= p.seq_len) return;
    const int parts = ncols / 4;
    const int rows = p.seq_len - len;
    bf16x4 z;
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = (__bf16)0.f;
    for (int e = threadIdx.x; e < rows * parts; e += kThreads) {
        const int t = len + e / parts;
        *reinterpret_cast<bf16x4*>(p.out + ob + size_t(t) * os + col0 + 4 * (e % parts)) = z;
    }
}

// The one-level scan: one workgroup per (sequence, value head, NT Dv tiles) walks every chunk
// of the sequence from the initial state.  The one-tile form keeps under 256 registers so that
// two workgroups share a compute unit.  PFW: at most one workgroup per compute unit, with the
// record prefetch wave.
// The register budget of two workgroups per compute unit (at most 256 VGPRs a lane) for every
// four-wave form: with one, the compiler spreads the two- and four-tile forms over VGPRs and
// AGPRs and copies the accumulators back and forth inside the chunk loop.
// The one- and two-tile prefetched scans at head dim 128 walk on eight waves (the eight-wave
// step) with the prefetch wave as a ninth, one workgroup per compute unit (its budget: 9 waves,
// at most three on a SIMD).  One tile: 128K scan 1.96 -> 1.92 ms against the four-wave walk
// with buffer loads; with plain loads the eight-wave walk was slower (2.03 ms).  Two tiles
// (each chunk's W, Q', K_dec and gamma loaded once for 32 state rows): GQA scan (64 chains)
// 110 -> 98 us against the four-wave two-tile walk.
template <int NT, int D, bool PFW>
constexpr bool scan_w8() { return PFW && NT <= 2 && D == 128; }
template <int NT, int D, bool PFW>
constexpr int scan_threads() { return scan_w8<NT, D, PFW>() ? 9 * 64 : (PFW ? kPfThreads : kThreads); }

template <int NT, int D, bool PFW>
__global__ __launch_bounds__((scan_threads<NT, D, PFW>()), (scan_w8<NT, D, PFW>() ? 1 : 2))
void kda_scan_kernel(Params p) {
    constexpr int BV = 16 * NT;
    constexpr int MW = HD<D>::MW;
    __shared__ __attribute__((aligned(16))) _Float16 sSh[BV * HD<D>::SLD];
    __shared__ __attribute__((aligned(16))) _Float16 sVh[BV * VN_LD];
    __shared__ __attribute__((aligned(16))) _Float16 sVl[BV * VN_LD];
    __shared__ __attribute__((aligned(16))) float sG[D];
    const ScanLds L{sSh, nullptr, sVh, sVl, sG};

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int q4 = lane >> 4;
    const int n16 = lane & 15;

    // XCD-aware decode: the Dv tiles of one (sequence, head) share blockIdx.x mod 8, so they
    // run on one XCD and share its L2 for the chunk operands they all read.
    const int pid = blockIdx.x;
    const int xcd = pid & 7, r8 = pid >> 3;
    const int bh = (r8 / p.scan_tiles) * 8 + xcd;
    const int tile = r8 % p.scan_tiles;
    if (bh >= p.batch * p.n_v) return;
    const int b = seq_by_rank(p, bh / p.n_v);
    const int h = bh % p.n_v;
    const int dv_tile0 = tile * NT;   // first 16-wide Dv tile of this workgroup

    int c0, len, slot0;
    seq_info(p, b, c0, len, slot0);
    const int nchunks = (len + kChunk - 1) / kChunk;
    size_t ob, os;
    row_geom(p, b, h, p.n_v, D, c0, ob, os);
    const int64_t rec0 = int64_t(slot0) * p.n_v + h;
    constexpr bool W8 = scan_w8<NT, D, PFW>();
    if constexpr (PFW) {
        if (w == (W8 ? 8 : 4)) {   // the prefetch wave: the setup barrier, then the walk's barriers
            RecPrefetch<D> pf;
            pf.init(p, tile, p.scan_tiles, dv_tile0, NT);
            if (nchunks > 1) pf.template touch<3>(rec0 + p.n_v);
            lds_barrier();
            prefetch_walk<D>(pf, rec0, p.n_v, 0, nchunks);
            pf.finish(p);
            return;
        }
    }

    const size_t st_base = (size_t(b) * p.n_v + h) * D * D;
    if constexpr (W8) {   // wave w holds Dk tile w of each of the workgroup's NT Dv tiles
        const int dk = 16 * w + 4 * q4;
        f32x4 S8[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int dv = 16 * (dv_tile0 + nt) + n16;
            S8[nt] = p.init ? *reinterpret_cast<const f32x4*>(p.init + st_base + size_t(dv) * D + dk)
                            : f32x4{0.f, 0.f, 0.f, 0.f};
            put_state_hi<D>(sSh, 16 * nt + n16, dk, S8[nt]);
        }
        lds_barrier();
        run_chunks8<true, OUT_FINAL, D, true, NT>(p, S8, L, rec0, 0, nchunks, len, ob, os,
                                                  dv_tile0);
        if (p.fin) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int dv = 16 * (dv_tile0 + nt) + n16;
                *reinterpret_cast<f32x4*>(p.fin + st_base + size_t(dv) * D + dk) = S8[nt];
            }
        }
        if (tid < kThreads) zero_rows_past_len(p, len, ob, os, 16 * dv_tile0, 16 * NT);
        return;
    }
    // state tile: S[mt][nt][i] = S[dv = 16(dv_tile0+nt) + n16][dk = 16(MW w+mt) + 4q4 + i]
    f32x4 S[MW][NT];
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int dv = 16 * (dv_tile0 + nt) + n16;
            const int dk = 16 * (MW * w + mt) + 4 * q4;
            S[mt][nt] = p.init ? *reinterpret_cast<const f32x4*>(p.init + st_base + size_t(dv) * D + dk)
                               : f32x4{0.f, 0.f, 0.f, 0.f};
            put_state_hi<D>(sSh, 16 * nt + n16, dk, S[mt][nt]);
        }
    lds_barrier();

    // split loads measured faster for the wider tiles, slower for the one-tile prefetched form,
    // which takes gamma through LDS instead
    constexpr bool SPLIT = NT > 1, GLDS = PFW && NT == 1;
    run_chunks<NT, D, SPLIT, GLDS>(p, S, L, rec0, 0, nchunks, len, ob, os, dv_tile0);

    if (p.fin) {
#pragma unroll
        for (int mt = 0; mt < MW; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int dv = 16 * (dv_tile0 + nt) + n16;
                const int dk = 16 * (MW * w + mt) + 4 * q4;
                *reinterpret_cast<f32x4*>(p.fin + st_base + size_t(dv) * D + dk) = S[mt][nt];
            }
    }
    zero_rows_past_len(p, len, ob, os, 16 * dv_tile0, 16 * NT);
}

// Segment pass of the two-level scan: 2 D/16 workgroups per (sequence, head, segment s >= 1),
// D/16 for segment 0.  The zero-start walk (D/16 workgroups, one 16-row Dv tile each) starts
// from S = 0 (from the initial state for s = 0) with U: the outputs of segment 0 are final,
// those of later segments go to O0, and the end state is N_s.  The identity walk (D/16
// workgroups from 16 identity rows each, without U) writes the columns of R = Q' P^T as its
// outputs and ends with the rows of P_s.  The walk runs on eight waves (the eight-wave step,
// scan_step8: two waves on every SIMD; one 16-row Dk tile of the state per wave at head dim
// 128, per X wave at 64).  Head dim 64: segment pass at 8K 17.9-18.2 -> 17.0-17.4 us against
// the four-wave walk.
template <int D>
constexpr int seg_waves() { return 8; }

template <int D>
__global__ __launch_bounds__(64 * seg_waves<D>(), 2) void kda_seg_kernel(Params p) {
    constexpr int NW = seg_waves<D>();
    constexpr int NDK = D / 16;                               // Dk tiles of the state
    constexpr int MW = NDK >= NW ? NDK / NW : 1, TILES = HD<D>::TILES;   // Dk tiles per wave
    const bool holds = int(threadIdx.x >> 6) < NDK;           // this wave holds a Dk tile
    __shared__ __attribute__((aligned(16))) _Float16 sSh[16 * HD<D>::SLD];
    __shared__ __attribute__((aligned(16))) _Float16 sVh[16 * VN_LD];
    __shared__ __attribute__((aligned(16))) _Float16 sVl[16 * VN_LD];
    __shared__ __attribute__((aligned(16))) float sG[D];
    const ScanLds L{sSh, nullptr, sVh, sVl, sG};

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int q4 = lane >> 4;
    const int n16 = lane & 15;

    // XCD-aware decode.  Both walks of a segment s >= 1 (2 D/16 workgroups, a "pair") run on
    // one XCD, so the segment's records are fetched into one L2 once; pair q = bh (seg_p - 1) +
    // s - 1 goes to XCD q mod 8.  The zero-start walks of segment 0 (D/16 workgroups, a
    // "single" per (sequence, head)) follow round-robin from the XCD after the last pair, so
    // that the XCDs receive nearly equal numbers of workgroups.
    const int pid = blockIdx.x;
    const int xcd = pid & 7, r8 = pid >> 3;
    const int n_bh = p.batch * p.n_v;
    const int np = n_bh * (p.seg_p - 1);           // pairs
    const int npx = (np + 7 - xcd) / 8;            // pairs on this XCD
    int bh, seg, tile;
    bool is_p;
    if (r8 < npx * 2 * TILES) {
        const int q = (r8 / (2 * TILES)) * 8 + xcd;
        const int slot = r8 % (2 * TILES);
        bh = q / (p.seg_p - 1);
        seg = q % (p.seg_p - 1) + 1;
        is_p = slot >= TILES;
        tile = slot % TILES;
    } else {
        const int r = r8 - npx * 2 * TILES;
        const int q = (xcd - np % 8 + 8) % 8 + 8 * (r / TILES);   // single q runs on XCD (np + q) mod 8
        if (q >= n_bh) return;
        bh = q;
        seg = 0;
        is_p = false;
        tile = r % TILES;
    }
    const int b = bh / p.n_v;
    const int h = bh % p.n_v;

    int c0, len, slot0;
    seq_info(p, b, c0, len, slot0);
    const int nchunks = (len + kChunk - 1) / kChunk;
    int cb, ce;
    segment_range(nchunks, p.seg_p, seg, cb, ce);
    size_t ob, os;
    row_geom(p, b, h, p.n_v, D, c0, ob, os);
    const int64_t rec0 = int64_t(slot0) * p.n_v + h;

    f32x4 S[MW][1];
    const size_t st_base = (size_t(b) * p.n_v + h) * D * D;
    const int row = 16 * tile + n16;   // state row (value channel, or identity row)
#pragma unroll
    for (int mt = 0; mt < MW; ++mt) {
        if (!holds) { S[mt][0] = f32x4{0.f, 0.f, 0.f, 0.f}; continue; }
        const int dk = 16 * (MW * w + mt) + 4 * q4;
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (is_p) {
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = (dk + i == row) ? 1.f : 0.f;
        } else if (seg == 0 && p.init) {
            x = *reinterpret_cast<const f32x4*>(p.init + st_base + size_t(row) * D + dk);
        }
        S[mt][0] = x;
        put_state_hi<D>(sSh, n16, dk, x);
    }
    lds_barrier();

    const size_t m = (size_t(bh) * p.seg_p + seg) * D * D;
    if (is_p) {
        run_chunks8<false, OUT_R, D>(p, S[0], L, rec0, cb, ce, len, ob, os, tile);
        // rows 16 tile .. of P_s, in fp16, into the combine's A fragments of P_s^T: element
        // P_s[16 tile + n16][16 M + 4 q4 + i] is lane (2 (tile & 1) + (n16 >> 3), 4 q4 + i),
        // entry n16 & 7, of fragment (M, tile >> 1)
        _Float16* pt = p.Pt + m;
        constexpr int KB = HD<D>::KB;
#pragma unroll
        for (int mt = 0; mt < MW; ++mt)
            if (holds)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int lp = (2 * (tile & 1) + (n16 >> 3)) * 16 + 4 * q4 + i;
                const int at = (((MW * w + mt) * KB + (tile >> 1)) * 64 + lp) * 8 + (n16 & 7);
                pt[at] = (_Float16)S[mt][0][i];
            }
    } else {
        if (seg == 0)
            run_chunks8<true, OUT_FINAL, D>(p, S[0], L, rec0, cb, ce, len, ob, os, tile);
        else
            run_chunks8<true, OUT_O0, D>(p, S[0], L, rec0, cb, ce, len, ob, os, tile);
#pragma unroll
        for (int mt = 0; mt < MW; ++mt)
            if (holds)
                *reinterpret_cast<f32x4*>(p.Nst + m + ((tile * TILES + MW * w + mt) * 64 + lane) * 4) =
                    S[mt][0];
        if (seg == 0) {   // S_in(1) = N_0 for the completion of segment 1 (combine pass layout)
            constexpr int KB = HD<D>::KB;
            __bf16* dst = p.Sin + (size_t(bh) * p.seg_p + 1) * D * D;
#pragma unroll
            for (int mt = 0; mt < MW; ++mt) {
                if (!holds) continue;
                const int M = MW * w + mt;
                const int lb = (2 * (M & 1) + (q4 >> 1)) * 16 + n16;
                *reinterpret_cast<bf16x4*>(dst + ((tile * KB + (M >> 1)) * 64 + lb) * 8 +
                                           4 * (q4 & 1)) = to_bf16x4(S[mt][0]);
            }
        }
    }
}

template <int D>
__device__ __forceinline__ void complete_record(const Params& p, int64_t rec, int seg_lo,
                                                int seg_hi, bf16x8* sR);

// Combine pass of the two-level scan: D/16 workgroups per (sequence, head), one 16-row Dv tile
// each, form S_in(1) = N_0 and S_in(s+1) = S_in(s) P_s + N_s and store every S_in(s) (bf16,
// for the completion pass).  With a final state it also keeps S_in(seg_p-1) in fp32, in the
// place of N_0 (whose rows only this workgroup reads, at its start): the last product,
// S_in(seg_p-1) P_last + N_last, runs in the completion pass beside the outputs, so that the
// outputs do not wait for it.  No step's operands depend on an earlier step, so they load two
// steps ahead, in three register sets (a load past the end rereads the last step's matrices,
// never used).  The register budget of two workgroups per compute unit (no AGPR copies).
template <int D>
__global__ __launch_bounds__(kThreads, 2) void kda_combine_kernel(Params p) {
    constexpr int MW = HD<D>::MW, KB = HD<D>::KB, TILES = HD<D>::TILES;
    __shared__ __attribute__((aligned(16))) _Float16 sSh[16 * HD<D>::SLD];
    __shared__ __attribute__((aligned(16))) _Float16 sSl[16 * HD<D>::SLD];
    const ScanLds L{sSh, sSl, nullptr, nullptr, nullptr};

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int q4 = lane >> 4;
    const int n16 = lane & 15;

    const int n_chain = (p.batch * p.n_v + 7) / 8 * 8 * TILES;   // chain workgroups, XCD padded
    if (int(blockIdx.x) >= n_chain) {   // segment 1's outputs: S_in(1) = N_0 is already stored
        __shared__ __attribute__((aligned(16))) bf16x8 sR[64 * D * 2 / 16];
        complete_record<D>(p, int64_t(blockIdx.x) - n_chain, 1, 1, sR);
        return;
    }
    const int pid = blockIdx.x;
    const int xcd = pid & 7, r8 = pid >> 3;
    const int bh = (r8 / TILES) * 8 + xcd;
    const int tile = r8 % TILES;
    if (bh >= p.batch * p.n_v) return;
    const int b = bh / p.n_v;
    const int h = bh % p.n_v;
    auto mat = [&](int s) { return (size_t(bh) * p.seg_p + s) * D * D; };

    const int last = p.seg_p - 2;   // steps 1 .. last: S_in(2) .. S_in(seg_p - 1)
    auto at = [&](int s) { return mat(s < last ? s : (last > 0 ? last : 1)); };
    f32x4 S[MW][1];
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
        S[mt][0] = *reinterpret_cast<const f32x4*>(p.Nst + mat(0) +
                                                   ((tile * TILES + MW * w + mt) * 64 + lane) * 4);
    CombFrags<1, D> c0f, c1f, c2f;
    load_comb<1, D>(p.Pt + at(1), p.Nst + at(1), tile, c0f);
    load_comb<1, D>(p.Pt + at(2), p.Nst + at(2), tile, c1f);
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
        put_state16<D>(sSh, sSl, n16, 16 * (MW * w + mt) + 4 * q4, S[mt][0]);
    lds_barrier();

    // S_in(s) in bf16 as the completion pass's A fragments: element S[16 tile + n16][16 M +
    // 4 q4 + i] is lane (2 (M & 1) + (q4 >> 1), n16), entries 4 (q4 & 1) + i, of fragment
    // (tile, M >> 1).  (The chain itself keeps S in fp32.)
    auto store_in = [&](int s) {
        if (s == 1) return;   // S_in(1) = N_0, stored by the segment pass
        __bf16* dst = p.Sin + mat(s);
#pragma unroll
        for (int mt = 0; mt < MW; ++mt) {
            const int M = MW * w + mt;
            const int lb = (2 * (M & 1) + (q4 >> 1)) * 16 + n16;
            const int off = ((tile * KB + (M >> 1)) * 64 + lb) * 8 + 4 * (q4 & 1);
            *reinterpret_cast<bf16x4*>(dst + off) = to_bf16x4(S[mt][0]);
        }
    };
    int s = 1;
    for (; s + 2 <= last; s += 3) {
        load_comb<1, D>(p.Pt + at(s + 2), p.Nst + at(s + 2), tile, c2f);
        store_in(s);
        combine_step<1, D>(c0f, S, L);
        load_comb<1, D>(p.Pt + at(s + 3), p.Nst + at(s + 3), tile, c0f);
        store_in(s + 1);
        combine_step<1, D>(c1f, S, L);
        load_comb<1, D>(p.Pt + at(s + 4), p.Nst + at(s + 4), tile, c1f);
        store_in(s + 2);
        combine_step<1, D>(c2f, S, L);
    }
    if (s <= last) {
        store_in(s);
        combine_step<1, D>(c0f, S, L);
        ++s;
    }
    if (s <= last) {
        store_in(s);
        combine_step<1, D>(c1f, S, L);
        ++s;
    }
    store_in(s);   // S_in(seg_p - 1)
    if (p.fin) {
#pragma unroll
        for (int mt = 0; mt < MW; ++mt)
            *reinterpret_cast<f32x4*>(p.Nst + mat(0) +
                                      ((tile * TILES + MW * w + mt) * 64 + lane) * 4) = S[mt][0];
    }

    int c0, len, slot0;
    seq_info(p, b, c0, len, slot0);
    size_t ob, os;
    row_geom(p, b, h, p.n_v, D, c0, ob, os);
    zero_rows_past_len(p, len, ob, os, 16 * tile, 16);
}

// Final state of one 16-row Dv tile of a (sequence, head): S_in(seg_p-1) P_last + N_last, with
// S_in(seg_p-1) in fp32 where the combine pass left it (the place of N_0).
template <int D>
__device__ __forceinline__ void final_state_step(const Params& p, int f, _Float16* lds) {
    constexpr int MW = HD<D>::MW, TILES = HD<D>::TILES;
    const int bh = f / TILES, tile = f % TILES;
    if (bh >= p.batch * p.n_v) return;
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int q4 = lane >> 4;
    const int n16 = lane & 15;
    const ScanLds L{lds, lds + 16 * HD<D>::SLD, nullptr, nullptr, nullptr};
    const size_t m0 = size_t(bh) * p.seg_p * D * D;
    const size_t ml = m0 + size_t(p.seg_p - 1) * D * D;
    f32x4 S[MW][1];
    CombFrags<1, D> cf;
    load_comb<1, D>(p.Pt + ml, p.Nst + ml, tile, cf);
#pragma unroll
    for (int mt = 0; mt < MW; ++mt) {
        S[mt][0] = *reinterpret_cast<const f32x4*>(p.Nst + m0 +
                                                   ((tile * TILES + MW * w + mt) * 64 + lane) * 4);
        put_state16<D>(L.sh, L.sl, n16, 16 * (MW * w + mt) + 4 * q4, S[mt][0]);
    }
    lds_barrier();
    combine_step<1, D>(cf, S, L);
    float* dst = p.fin + size_t(bh) * D * D + size_t(16 * tile + n16) * D;
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
        *reinterpret_cast<f32x4*>(dst + 16 * (MW * w + mt) + 4 * q4) = S[mt][0];
}

// Completion pass of the two-level scan: one workgroup per record of a chunk in segment
// s >= 1, out = O0 + R S_in(s)^T from bf16 S_in, R and O0 with fp32 sums (as O^T = S_in R^T:
// the accumulator holds four consecutive value channels of one token per lane).  Wave w takes Dv
// tiles D/64 w .. of all 64 tokens.  R, which every wave multiplies, is read from HBM once into
// LDS; every operand is loaded before the first output is stored.  The workgroups after the
// records form the final states (final_state_step), one per 16-row Dv tile of each (sequence,
// head).
// Output completion of the chunk record `rec` when its segment lies in [seg_lo, seg_hi]:
// out = O0 + R S_in(s)^T (the completion pass's workgroups and, for segment 1, whose S_in is
// N_0 from the segment pass, extra workgroups of the combine pass).  sR: 64 x D bf16 of LDS.
template <int D>
__device__ __forceinline__ void complete_record(const Params& p, int64_t rec, int seg_lo,
                                                int seg_hi, bf16x8* sR) {
    constexpr int KB = HD<D>::KB, NTW = D / 64;
    constexpr int R_U4 = 64 * D * 2 / 16;   // R in 16-byte units
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int q4 = lane >> 4;
    const int n16 = lane & 15;
    const unsigned slot_u = unsigned(rec) / unsigned(p.n_v);   // records stay below 2^31
    const int slot = int(slot_u);
    const int h = int(unsigned(rec) - slot_u * unsigned(p.n_v));
    const int b = slot_batch(p, slot);
    int c0, len, slot0;
    seq_info(p, b, c0, len, slot0);
    const int j = slot - slot0;
    if (j < 0 || j * kChunk >= len) return;   // an unused slot
    const int nchunks = (len + kChunk - 1) / kChunk;
    const int seg = int(unsigned(j) / ((unsigned(nchunks) + p.seg_p - 1) / unsigned(p.seg_p)));
    if (seg < seg_lo || seg > seg_hi) return;
    size_t ob, os;
    row_geom(p, b, h, p.n_v, D, c0, ob, os);

    const __bf16* sin = p.Sin + ((size_t(b) * p.n_v + h) * p.seg_p + seg) * D * D;
    const __bf16* o0 = p.O0 + size_t(rec) * (64 * D);
    const __bf16* rr = p.Rf + size_t(rec) * (64 * D);

    bf16x8 ah[NTW][KB];                // S_in[16 nt + n16][32 kb + 8 q4 ..]
    bf16x4 ob4[4][NTW];                // O0[16 tt + n16][16 nt + 4 q4 ..]
    {
        bf16x8 x[R_U4 / kThreads];
#pragma unroll
        for (int u = 0; u < R_U4 / kThreads; ++u)
            x[u] = *reinterpret_cast<const bf16x8*>(rr + size_t(u * kThreads + tid) * 8);
#pragma unroll
        for (int u = 0; u < R_U4 / kThreads; ++u) sR[u * kThreads + tid] = x[u];
    }
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            ah[i][kb] = *reinterpret_cast<const bf16x8*>(
                sin + (((NTW * w + i) * KB + kb) * 64 + lane) * 8);
        }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < NTW; ++i)
            ob4[tt][i] = *reinterpret_cast<const bf16x4*>(o0 + (((NTW * w + i) * 4 + tt) * 64 + lane) * 4);
    __syncthreads();
    f32x4 acc[4][NTW];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < NTW; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[tt][i][r] = (float)ob4[tt][i][r];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const bf16x8 br = sR[(tt * KB + kb) * 64 + lane];   // R[16 tt + n16][32 kb + 8 q4 ..]
#pragma unroll
            for (int i = 0; i < NTW; ++i) acc[tt][i] = mfma(ah[i][kb], br, acc[tt][i]);
        }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int tok = j * kChunk + 16 * tt + n16;
        if (tok < len) {
#pragma unroll
            for (int i = 0; i < NTW; ++i)
                *reinterpret_cast<bf16x4*>(p.out + ob + size_t(tok) * os +
                                           16 * (NTW * w + i) + 4 * q4) = to_bf16x4(acc[tt][i]);
        }
    }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void kda_out_kernel(Params p) {
    constexpr int R_U4 = 64 * D * 2 / 16;   // R in 16-byte units
    static_assert(R_U4 * 16 >= 2 * 16 * HD<D>::SLD * 2, "the state tiles fit the R buffer");
    __shared__ __attribute__((aligned(16))) bf16x8 sR[R_U4];
    const int64_t rec = blockIdx.x;
    const int64_t n_rec = int64_t(p.intra_units) * p.group;
    if (rec >= n_rec) {
        if (p.fin) final_state_step<D>(p, int(rec - n_rec), reinterpret_cast<_Float16*>(sR));
        return;
    }
    complete_record<D>(p, rec, 2, p.seg_p - 1, sR);   // segment 1 runs in the combine pass
}

// Stages of one call, each one kernel (empty when the plan does not enqueue it): intra, then
// either the one-level scan or the segment, combine and completion passes.
constexpr int kStages = 5;
enum Stage { ST_INTRA = 0, ST_SEG = 1, ST_COMB = 2, ST_OUT = 3, ST_SCAN = 4 };

// One kernel launch.  With events, the dispatch itself records e0 when the kernel starts and
// e1 when it ends (hipExtLaunchKernel), so no marker packet sits between the kernels.
kda_status launch_kernel(const void* kernel, unsigned grid, unsigned threads, hipStream_t stream,
                         hipEvent_t e0, hipEvent_t e1, Params& p) {
    void* args[] = {&p};
    if (hipExtLaunchKernel(kernel, dim3(grid), dim3(threads), args, 0, stream, e0, e1, 0) !=
        hipSuccess)
        return KDA_ERR_HIP;
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// Every kernel variant the library holds, named by its template arguments.  The plan picks one
// per stage by name (stage_kernels), so the names a plan query reports are exactly the kernels a
// call launches.
struct Variant {
    const char* name;
    const void* fn;
    unsigned threads;
};
#define KDA_VARIANT(kern, threads, ...) \
    {#kern "<" #__VA_ARGS__ ">", reinterpret_cast<const void*>(&kern<__VA_ARGS__>), threads}
const Variant kVariants[] = {
    KDA_VARIANT(kda_intra_kernel, kThreads, 0,128,1),
    KDA_VARIANT(kda_intra_kernel, 2 * kThreads, 0,128,2),
    KDA_VARIANT(kda_intra_kernel, kThreads, 1,128,1),
    KDA_VARIANT(kda_intra_kernel, 2 * kThreads, 1,128,2),
    KDA_VARIANT(kda_intra_kernel, kThreads, 0,64,1),
    KDA_VARIANT(kda_intra_kernel, 2 * kThreads, 0,64,2),
    KDA_VARIANT(kda_intra_kernel, kThreads, 1,64,1),
    KDA_VARIANT(kda_intra_kernel, 2 * kThreads, 1,64,2),
    KDA_VARIANT(kda_intra_kernel, kThreads, 2,128,1),
    KDA_VARIANT(kda_intra_kernel, 2 * kThreads, 2,128,2),
    KDA_VARIANT(kda_intra_kernel, kThreads, 2,64,1),
    KDA_VARIANT(kda_intra_kernel, 2 * kThreads, 2,64,2),
    KDA_VARIANT(kda_seg_kernel, 64 * seg_waves<128>(), 128),
    KDA_VARIANT(kda_seg_kernel, 64 * seg_waves<64>(), 64),
    KDA_VARIANT(kda_combine_kernel, kThreads, 128),
    KDA_VARIANT(kda_combine_kernel, kThreads, 64),
    KDA_VARIANT(kda_out_kernel, kThreads, 128),
    KDA_VARIANT(kda_out_kernel, kThreads, 64),
    KDA_VARIANT(kda_scan_kernel, (scan_threads<1, 128, true>()), 1,128,true),
    KDA_VARIANT(kda_scan_kernel, (scan_threads<2, 128, true>()), 2,128,true),
    KDA_VARIANT(kda_scan_kernel, kThreads, 2,128,false),
    KDA_VARIANT(kda_scan_kernel, kThreads, 4,128,false),
    KDA_VARIANT(kda_scan_kernel, (scan_threads<1, 64, true>()), 1,64,true),
    KDA_VARIANT(kda_scan_kernel, (scan_threads<2, 64, true>()), 2,64,true),
    KDA_VARIANT(kda_scan_kernel, kThreads, 1,64,false),
    KDA_VARIANT(kda_scan_kernel, kThreads, 2,64,false),
    KDA_VARIANT(kda_scan_kernel, kThreads, 4,64,false),
};
#undef KDA_VARIANT
constexpr int kNumVariants = int(sizeof(kVariants) / sizeof(kVariants[0]));
constexpr int kNameCap = 64;

// Name of the kernel each stage of `plan` launches; an empty name for a stage the plan skips.
void stage_kernels(const Plan& plan, uint32_t flags, char (&names)[kStages][kNameCap]) {
    for (auto& n : names) n[0] = '\0';
    const int gm = (flags & KDA_RAW_GATE) ? 2 : (flags & KDA_SCALAR_GATE) ? 1 : 0;
    std::snprintf(names[ST_INTRA], kNameCap, "kda_intra_kernel<%d,%d,%d>", gm, plan.d,
                  plan.intra_hv);
    if (plan.seg_p > 1) {
        std::snprintf(names[ST_SEG], kNameCap, "kda_seg_kernel<%d>", plan.d);
        std::snprintf(names[ST_COMB], kNameCap, "kda_combine_kernel<%d>", plan.d);
        std::snprintf(names[ST_OUT], kNameCap, "kda_out_kernel<%d>", plan.d);
    } else {
        std::snprintf(names[ST_SCAN], kNameCap, "kda_scan_kernel<%d,%d,%s>", plan.scan_nt,
                      plan.d, plan.scan_pf ? "true" : "false");
    }
}

const Variant* find_variant(const char* name) {
    for (const Variant& v : kVariants)
        if (std::strcmp(v.name, name) == 0) return &v;
    return nullptr;
}

// `gate` is the raw-gate activation (kda_chunk_fwd_raw_gate; g then points at the raw bf16
// gate) or NULL (g is the fp32 activated gate).  The shape's KDA_RAW_GATE flag must agree.
kda_status launch(const kda_shape* shape, const void* q, const void* k, const void* v,
                  const void* g, const kda_raw_gate* gate, const void* beta,
                  const float* initial_state, const int32_t* cu_seqlens, void* out,
                  float* final_state, void* workspace, size_t workspace_bytes,
                  hipStream_t stream, hipEvent_t* ev, int n_ev) {
    Plan plan;
    kda_status st = make_plan(shape, &plan);
    if (st != KDA_OK) return st;
    if (((shape->flags & KDA_RAW_GATE) != 0) != (gate != nullptr)) return KDA_ERR_INVALID_ARG;
    st = check_call(shape, plan, q, k, v, g, gate, beta, initial_state, cu_seqlens, out,
                    final_state, workspace, workspace_bytes);
    if (st != KDA_OK) return st;
    if (ev && n_ev < 2 * kStages) return KDA_ERR_INVALID_ARG;

    Params p;
    p.q = static_cast<const __bf16*>(q);
    p.k = static_cast<const __bf16*>(k);
    p.v = static_cast<const __bf16*>(v);
    p.g = gate ? nullptr : static_cast<const float*>(g);
    p.graw = gate ? static_cast<const __bf16*>(g) : nullptr;
    p.a_log = gate ? gate->a_log : nullptr;
    p.dt_bias = gate ? gate->dt_bias : nullptr;
    p.lower_bound = gate ? gate->lower_bound : 0.f;
    p.beta = static_cast<const __bf16*>(beta);
    p.init = initial_state;
    p.cu = cu_seqlens;
    p.out = static_cast<__bf16*>(out);
    p.fin = final_state;
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    p.Wf = reinterpret_cast<_Float16*>(ws + plan.off_w);
    p.Qf = reinterpret_cast<_Float16*>(ws + plan.off_q);
    p.Kf = reinterpret_cast<_Float16*>(ws + plan.off_k);
    p.Uf = reinterpret_cast<_Float16*>(ws + plan.off_u);
    p.Of = reinterpret_cast<__bf16*>(ws + plan.off_o);
    p.Gf = reinterpret_cast<float*>(ws + plan.off_g);
    p.layout = plan.layout;
    p.batch = plan.batch;
    p.seq_len = plan.seq_len;
    p.n_qk = plan.n_qk;
    p.n_v = plan.n_v;
    p.group = plan.group;
    p.nc_max = plan.nc_max;
    p.scan_tiles = plan.scan_tiles;
    p.seg_p = plan.seg_p;
    const bool two = plan.seg_p > 1;
    p.Pt = two ? reinterpret_cast<_Float16*>(ws + plan.off_pt) : nullptr;
    p.Nst = two ? reinterpret_cast<float*>(ws + plan.off_n) : nullptr;
    p.Sin = two ? reinterpret_cast<__bf16*>(ws + plan.off_sin) : nullptr;
    p.O0 = two ? reinterpret_cast<__bf16*>(ws + plan.off_o0) : nullptr;
    p.Rf = two ? reinterpret_cast<__bf16*>(ws + plan.off_r) : nullptr;
    p.scale = shape->scale;
    p.flags = shape->flags;
    p.intra_units = int(plan.n_records / plan.group);

    char names[kStages][kNameCap];
    stage_kernels(plan, shape->flags, names);
    const int64_t grid[kStages] = {plan.intra_blocks, plan.seg_blocks, plan.comb_blocks,
                                   plan.out_blocks, plan.scan_blocks};
    (void)hipGetLastError();  // clear a stale error so the checks below see only ours
    for (int s = 0; s < kStages; ++s) {
        if (names[s][0]) {
            const Variant* var = find_variant(names[s]);
            if (!var) return KDA_ERR_UNSUPPORTED;
            st = launch_kernel(var->fn, unsigned(grid[s]), var->threads, stream,
                               ev ? ev[2 * s] : nullptr, ev ? ev[2 * s + 1] : nullptr, p);
            if (st != KDA_OK) return st;
        } else if (ev && (hipEventRecord(ev[2 * s], stream) != hipSuccess ||
                          hipEventRecord(ev[2 * s + 1], stream) != hipSuccess)) {
            // a stage the plan skips: its two events back to back
            return KDA_ERR_HIP;
        }
    }
    return KDA_OK;
}

// ---------------------------------------------------------------------------------------------
// Allocation-free entry point
// ---------------------------------------------------------------------------------------------
//
// For callers that cannot allocate device memory (HIP graph capture, tight serving loops):
// the workspace lives in a file-scope device array, one copy per GPU the library runs on, held
// until the process ends.  Host code never passes the array's name to a kernel (on the host it
// is only a stand-in for the symbol): its device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and that address is what the kernels get.
// Every call on one GPU shares the array; nothing in it has to start at zero (every workspace
// element a kernel reads was written by an earlier kernel of the same call), but calls that
// overlap in time on one GPU (two streams, two threads) race on it.
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

kda_status scratch_of_current_device(void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KDA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KDA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return KDA_OK;
}

}  // namespace kda

extern "C" {

kda_status kda_chunk_fwd_workspace(const kda_shape* shape, size_t* bytes) {
    if (!bytes) return KDA_ERR_INVALID_ARG;
    kda::Plan plan;
    const kda_status st = kda::make_plan(shape, &plan);
    if (st != KDA_OK) return st;
    *bytes = plan.total;
    return KDA_OK;
}

kda_status kda_chunk_fwd(const kda_shape* shape, const void* q, const void* k, const void* v,
                         const float* g, const void* beta, const float* initial_state,
                         const int32_t* cu_seqlens, void* out, float* final_state,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return kda::launch(shape, q, k, v, g, nullptr, beta, initial_state, cu_seqlens, out,
                       final_state, workspace, workspace_bytes, stream, nullptr, 0);
}

kda_status kda_chunk_fwd_raw_gate(const kda_shape* shape, const void* q, const void* k,
                                  const void* v, const void* g_raw, const void* beta,
                                  const kda_raw_gate* gate, const float* initial_state,
                                  const int32_t* cu_seqlens, void* out, float* final_state,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!gate) return KDA_ERR_INVALID_ARG;
    return kda::launch(shape, q, k, v, g_raw, gate, beta, initial_state, cu_seqlens, out,
                       final_state, workspace, workspace_bytes, stream, nullptr, 0);
}

kda_status kda_chunk_fwd_raw_gate_timed(const kda_shape* shape, const void* q, const void* k,
                                        const void* v, const void* g_raw, const void* beta,
                                        const kda_raw_gate* gate, const float* initial_state,
                                        const int32_t* cu_seqlens, void* out, float* final_state,
                                        void* workspace, size_t workspace_bytes,
                                        hipStream_t stream, hipEvent_t* stage_events,
                                        int32_t n_stage_events) {
    if (!gate || !stage_events || n_stage_events < 2 * kda::kStages) return KDA_ERR_INVALID_ARG;
    return kda::launch(shape, q, k, v, g_raw, gate, beta, initial_state, cu_seqlens, out,
                       final_state, workspace, workspace_bytes, stream, stage_events,
                       n_stage_events);
}

kda_status kda_chunk_fwd_noalloc(const kda_shape* shape, const void* q, const void* k,
                                 const void* v, const float* g, const void* beta,
                                 const float* initial_state, const int32_t* cu_seqlens, void* out,
                                 float* final_state, hipStream_t stream) {
    kda::Plan plan;
    const kda_status st = kda::make_plan(shape, &plan);
    if (st != KDA_OK) return st;
    if (plan.total > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_WORKSPACE;
    void* ws = nullptr;
    if (kda::scratch_of_current_device(&ws) != KDA_OK) return KDA_ERR_HIP;
    return kda::launch(shape, q, k, v, g, nullptr, beta, initial_state, cu_seqlens, out,
                       final_state, ws, KDA_NOALLOC_SCRATCH_BYTES, stream, nullptr, 0);
}

kda_status kda_chunk_fwd_timed(const kda_shape* shape, const void* q, const void* k,
                               const void* v, const float* g, const void* beta,
                               const float* initial_state, const int32_t* cu_seqlens, void* out,
                               float* final_state, void* workspace, size_t workspace_bytes,
                               hipStream_t stream, hipEvent_t* stage_events,
                               int32_t n_stage_events) {
    if (!stage_events || n_stage_events < 2 * kda::kStages) return KDA_ERR_INVALID_ARG;
    return kda::launch(shape, q, k, v, g, nullptr, beta, initial_state, cu_seqlens, out,
                       final_state, workspace, workspace_bytes, stream, stage_events,
                       n_stage_events);
}

int32_t kda_num_stages(void) { return kda::kStages; }

kda_status kda_chunk_fwd_plan(const kda_shape* shape, uint32_t* stage_mask, int32_t* segments) {
    kda::Plan plan;
    const kda_status st = kda::make_plan(shape, &plan);
    if (st != KDA_OK) return st;
    const bool two = plan.seg_p > 1;
    if (stage_mask)
        *stage_mask = (1u << kda::ST_INTRA) |
                      (two ? (1u << kda::ST_SEG) | (1u << kda::ST_COMB) | (1u << kda::ST_OUT)
                           : (1u << kda::ST_SCAN));
    if (segments) *segments = plan.seg_p;
    return KDA_OK;
}

kda_status kda_chunk_fwd_plan_kernels(const kda_shape* shape, char* names, size_t capacity) {
    if (!names) return KDA_ERR_INVALID_ARG;
    kda::Plan plan;
    const kda_status st = kda::make_plan(shape, &plan);
    if (st != KDA_OK) return st;
    char stage[kda::kStages][kda::kNameCap];
    kda::stage_kernels(plan, shape->flags, stage);
    size_t need = 1;   // the NUL, and one ';' between two names
    int count = 0;
    for (const auto& n : stage)
        if (n[0]) need += std::strlen(n) + (count++ ? 1 : 0);
    if (capacity < need) return KDA_ERR_INVALID_ARG;
    names[0] = '\0';
    for (const auto& n : stage) {
        if (!n[0]) continue;
        if (names[0]) std::strcat(names, ";");
        std::strcat(names, n);
    }
    return KDA_OK;
}

int32_t kda_num_kernel_variants(void) { return kda::kNumVariants; }

const char* kda_kernel_variant(int32_t i) {
    return (i >= 0 && i < kda::kNumVariants) ? kda::kVariants[i].name : nullptr;
}

const char* kda_stage_name(int32_t stage) {
    switch (stage) {
    case kda::ST_INTRA: return "kda_intra_kernel";
    case kda::ST_SEG: return "kda_seg_kernel";
    case kda::ST_COMB: return "kda_combine_kernel";
    case kda::ST_OUT: return "kda_out_kernel";
    case kda::ST_SCAN: return "kda_scan_kernel";
    default: return "unknown stage";
    }
}

const char* kda_status_str(kda_status status) {
    switch (status) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
    default: return "unknown kda_status";
    }
}

int32_t kda_version(void) { return 100; }

}  // extern "C"
