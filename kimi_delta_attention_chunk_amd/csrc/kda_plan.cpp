// kda_plan.cpp -- host-side validation and planning for the KDA chunked forward.
//
// The accepted argument space follows the FlashKDA README, section 约束说明: Dk = Dv = 128 (and
// here also Dk = Dv = 64),
// B >= 1, stored length > 0, layouts BNSD / BSND / TND, 1 <= Nqk <= Nv with Nv % Nqk == 0,
// TND needs an int32 cu_seqlens of B+1 entries, and final_state is a new tensor (here: it must
// not overlap initial_state).  Only shapes and pointers are inspected; device data is never read.
#include "kda_plan.h"

#include <cmath>
#include <limits>

namespace kda {

namespace {

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

}  // namespace

kda_status make_plan(const kda_shape* s, Plan* plan) {
    if (!s || !plan) return KDA_ERR_INVALID_ARG;
    if (s->layout < KDA_LAYOUT_BNSD || s->layout > KDA_LAYOUT_TND) return KDA_ERR_INVALID_ARG;
    if (s->batch < 1 || s->seq_len < 1) return KDA_ERR_INVALID_ARG;
    if (s->n_qk < 1 || s->n_v < s->n_qk || s->n_v % s->n_qk != 0) return KDA_ERR_INVALID_ARG;
    if (s->d_k < 1 || s->d_v < 1) return KDA_ERR_INVALID_ARG;
    if (s->d_k != s->d_v || !head_dim_ok(s->d_k)) return KDA_ERR_UNSUPPORTED;
    if (!std::isfinite(s->scale)) return KDA_ERR_INVALID_ARG;
    if (s->flags & ~uint32_t(KDA_QK_L2NORM | KDA_BETA_SIGMOID | KDA_SCALAR_GATE | KDA_RAW_GATE))
        return KDA_ERR_INVALID_ARG;
    // the raw gate (FlashKDA README, 参数说明) has one value per key channel
    if ((s->flags & KDA_RAW_GATE) && (s->flags & KDA_SCALAR_GATE)) return KDA_ERR_UNSUPPORTED;
    if (s->layout == KDA_LAYOUT_TND && s->seq_len < s->batch) return KDA_ERR_INVALID_ARG;

    Plan p;
    p.layout = s->layout;
    p.d = s->d_k;
    p.batch = s->batch;
    p.seq_len = s->seq_len;
    p.n_qk = s->n_qk;
    p.n_v = s->n_v;
    p.group = s->n_v / s->n_qk;
    if (s->layout == KDA_LAYOUT_TND) {
        // chunk j of sequence b lives in slot floor(cu[b]/64) + b + j: distinct for distinct
        // (b, j) and below floor(T/64) + N for every valid prefix sum
        p.nc_max = 0;
        p.n_slots = int64_t(s->seq_len) / kChunk + s->batch;
    } else {
        p.nc_max = int((int64_t(s->seq_len) + kChunk - 1) / kChunk);
        p.n_slots = int64_t(s->batch) * p.nc_max;
    }
    // one intra workgroup per record: more than 2^31 - 1 records cannot be launched (checked
    // here, before any product that could overflow)
    if (double(p.n_slots) * double(s->n_v) >= double(std::numeric_limits<int32_t>::max()))
        return KDA_ERR_UNSUPPORTED;
    p.n_records = p.n_slots * s->n_v;
    // intra grid: units (chunk slot, q/k head) padded to a multiple of 8, times the group
    p.intra_blocks = (p.n_records / p.group + 7) / 8 * 8 * p.group;
    // When the whole intra grid is resident at once (at most two workgroups per compute unit),
    // a workgroup's latency is the stage's time, and eight waves (two per token block) shorten
    // it (measured: 256-token call -6 %, 8K tokens x 3 or 4 heads -2 %); larger grids run in
    // rounds, where the four-wave form, two (three at head dim 64) per compute unit, overlaps
    // one's memory phases with another's arithmetic.
    p.intra_hv = p.intra_blocks <= 512 ? 2 : 1;
    // Each scan workgroup streams a whole chunk record per step whatever its Dv width, so a
    // wider tile cuts the bytes streamed per unit of work; it is taken only while enough
    // workgroups remain to occupy all 256 compute units of an MI355X.
    const int64_t bh = int64_t(s->batch) * s->n_v;
    const int tiles = p.d / 16;   // 16-row Dv tiles per head
    p.scan_nt = 1;
    for (int nt = 4; nt >= 2; nt /= 2)
        if (bh * (tiles / nt) >= 256) { p.scan_nt = nt; break; }
    // At head dim 128, 33..63 chains would take 264..504 one-tile workgroups, two per compute
    // unit; as 132..252 two-tile workgroups with the record prefetch wave they run one per unit
    // on the eight-wave walk, which loads each chunk's shared operands once for both tiles
    // (measured at 8K tokens: 48 heads scan 285 -> 171 us, 40 heads 276 -> 167 us).
    if (p.scan_nt == 1 && p.d == 128 && bh * tiles > 256) p.scan_nt = 2;
    // Few (sequence, head) chains leave most compute units idle through a long sequential scan.
    // Then each sequence is cut into seg_p segments and every segment is walked at once: from
    // a zero state (from the initial state for segment 0), giving its end state N_s and the
    // outputs O0 of its chunks, and from the identity, giving its transfer matrix P_s and the
    // queries R = Q' P^T carried back to the segment start (d/16 + d/16 workgroups per
    // segment).  A short combine then forms S_in(s) = S_in(s-1) P_{s-1} + N_{s-1}, and the
    // outputs of segment s >= 1 are completed in parallel as O0 + R S_in(s)^T.  seg_p is the
    // largest count whose segment pass fits 256 workgroups, with at least 8 chunks per
    // segment.
    p.seg_p = 1;
    if (bh * tiles < 256) {
        const int64_t nc_est = (s->layout == KDA_LAYOUT_TND)
                                   ? (int64_t(s->seq_len) / s->batch + kChunk - 1) / kChunk
                                   : p.nc_max;
        int64_t sp = (256 / (bh * tiles) + 1) / 2;
        if (sp > nc_est / 8) sp = nc_est / 8;
        if (sp > 16) sp = 16;
        if (sp >= 2) p.seg_p = int(sp);
    }
    if (p.seg_p > 1) p.scan_nt = 1;
    p.scan_tiles = tiles / p.scan_nt;
    const int64_t bh8 = (bh + 7) / 8 * 8;
    if (p.seg_p > 1) {
        p.scan_blocks = 0;
        // per XCD x: its pairs ((np + 7 - x) / 8, 2 tiles workgroups each), then its singles
        // (segment 0 of sequence-head q runs on XCD (np + q) mod 8, tiles workgroups each)
        const int64_t np = bh * (p.seg_p - 1);
        int64_t rows = 0;
        for (int x = 0; x < 8; ++x) {
            const int64_t npx = (np + 7 - x) / 8;
            const int64_t q0 = (x - np % 8 + 8) % 8;   // first single on XCD x
            const int64_t nsx = q0 < bh ? (bh - q0 + 7) / 8 : 0;
            const int64_t r = npx * 2 * tiles + nsx * tiles;
            rows = r > rows ? r : rows;
        }
        p.seg_blocks = rows * 8;
        p.comb_blocks = bh8 * tiles + p.n_records;   // chains, then segment-1 outputs
        p.out_blocks = p.n_records + bh * tiles;   // records, then final-state tiles
    } else {
        p.scan_blocks = bh8 * p.scan_tiles;
        // a prefetch wave costs the second workgroup per compute unit: only when one per unit
        // is all there is, and not for the four-tile form (its registers would not fit two
        // waves per SIMD)
        p.scan_pf = bh * p.scan_tiles <= 256 && p.scan_nt <= 2;
    }
    const int64_t max_grid = std::numeric_limits<int32_t>::max();
    if (p.intra_blocks > max_grid || p.scan_blocks > max_grid || p.seg_blocks > max_grid ||
        p.comb_blocks > max_grid || p.out_blocks > max_grid)
        return KDA_ERR_UNSUPPORTED;

    // element counts of the largest tensors must fit the 64-bit offsets used on the device
    const double tokens = (s->layout == KDA_LAYOUT_TND) ? double(s->seq_len)
                                                        : double(s->batch) * s->seq_len;
    // (below 2^60 elements, so byte counts of every tensor, fp32 g included, stay below 2^62)
    if (tokens * s->n_v * p.d >= 1152921504606846976.0) return KDA_ERR_UNSUPPORTED;
    // the 64 output rows of one chunk are one buffer-store region with 32-bit byte offsets
    if (int64_t(kChunk) * s->n_v * p.d * 2 >= (int64_t(1) << 31)) return KDA_ERR_UNSUPPORTED;

    const size_t n = size_t(p.n_records);
    const int d = p.d;
    size_t off = 0;
    p.off_w = off; off = align_up(off + n * rec_w_bytes(d), 256);
    p.off_q = off; off = align_up(off + n * rec_q_bytes(d), 256);
    p.off_k = off; off = align_up(off + n * rec_k_bytes(d), 256);
    p.off_u = off; off = align_up(off + n * rec_u_bytes(d), 256);
    p.off_o = off; off = align_up(off + n * rec_o_bytes(d), 256);
    p.off_g = off; off = align_up(off + n * rec_g_bytes(d), 256);
    if (p.seg_p > 1) {
        const size_t mats = size_t(bh) * p.seg_p * d * d * sizeof(float);
        const size_t rows = n * kChunk * d * 2;   // bf16
        p.off_pt = off; off = align_up(off + mats / 2, 256);   // fp16
        p.off_n = off; off = align_up(off + mats, 256);
        p.off_sin = off; off = align_up(off + mats / 2, 256);   // bf16
        p.off_o0 = off; off = align_up(off + rows, 256);
        p.off_r = off; off = align_up(off + rows, 256);
    }
    p.total = off;
    *plan = p;
    return KDA_OK;
}

kda_status check_call(const kda_shape* s, const Plan& p, const void* q, const void* k,
                      const void* v, const void* g, const kda_raw_gate* gate, const void* beta,
                      const float* initial_state, const int32_t* cu_seqlens, const void* out,
                      const float* final_state, const void* workspace,
                      size_t workspace_bytes) {
    if (!q || !k || !v || !g || !beta || !out) return KDA_ERR_INVALID_ARG;
    if (gate) {   // raw-gate activation parameters (FlashKDA README, 约束说明: lower_bound in [-5, 0])
        if (!gate->a_log || !gate->dt_bias) return KDA_ERR_INVALID_ARG;
        if (!aligned(gate->a_log, 4) || !aligned(gate->dt_bias, 16)) return KDA_ERR_INVALID_ARG;
        if (!(gate->lower_bound >= -5.0f && gate->lower_bound <= 0.0f)) return KDA_ERR_INVALID_ARG;
    }
    if (s->layout == KDA_LAYOUT_TND && !cu_seqlens) return KDA_ERR_INVALID_ARG;
    const void* ptrs16[] = {q, k, v, g, out};
    for (const void* ptr : ptrs16)
        if (!aligned(ptr, 16)) return KDA_ERR_INVALID_ARG;
    if (!aligned(beta, 2)) return KDA_ERR_INVALID_ARG;
    if (initial_state && !aligned(initial_state, 16)) return KDA_ERR_INVALID_ARG;
    if (final_state && !aligned(final_state, 16)) return KDA_ERR_INVALID_ARG;
    if (cu_seqlens && !aligned(cu_seqlens, 4)) return KDA_ERR_INVALID_ARG;
    const size_t state_bytes = size_t(p.batch) * p.n_v * p.d * p.d * sizeof(float);
    if (initial_state && final_state &&
        overlap(initial_state, state_bytes, final_state, state_bytes))
        return KDA_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < p.total) return KDA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return KDA_ERR_WORKSPACE;

    // nothing the call writes (out, final_state, the workspace it uses) may overlap anything
    // else it reads or writes
    const size_t tokens = (s->layout == KDA_LAYOUT_TND) ? size_t(s->seq_len)
                                                        : size_t(s->batch) * s->seq_len;
    const size_t per_v = tokens * p.n_v;
    const bool sg = (s->flags & KDA_SCALAR_GATE) != 0;
    struct Region {
        const void* ptr;
        size_t bytes;
        bool written;
    };
    const Region r[] = {
        {q, tokens * p.n_qk * p.d * 2, false},
        {k, tokens * p.n_qk * p.d * 2, false},
        {v, per_v * p.d * 2, false},
        {g, per_v * (sg ? 1 : p.d) * (gate ? 2 : sizeof(float)), false},
        {gate ? gate->a_log : nullptr, gate ? size_t(p.n_v) * sizeof(float) : 0, false},
        {gate ? gate->dt_bias : nullptr, gate ? size_t(p.n_v) * p.d * sizeof(float) : 0, false},
        {beta, per_v * 2, false},
        {initial_state, initial_state ? state_bytes : 0, false},
        {cu_seqlens, cu_seqlens ? (size_t(s->batch) + 1) * sizeof(int32_t) : 0, false},
        {out, per_v * p.d * 2, true},
        {final_state, final_state ? state_bytes : 0, true},
        {workspace, p.total, true},
    };
    constexpr int nr = sizeof(r) / sizeof(r[0]);
    for (int i = 0; i < nr; ++i)
        for (int j = i + 1; j < nr; ++j)
            if ((r[i].written || r[j].written) && r[i].bytes && r[j].bytes &&
                overlap(r[i].ptr, r[i].bytes, r[j].ptr, r[j].bytes))
                return KDA_ERR_INVALID_ARG;
    return KDA_OK;
}

}  // namespace kda
