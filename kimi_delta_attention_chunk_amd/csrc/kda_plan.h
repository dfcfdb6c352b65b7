// kda_plan.h -- host-side argument validation, chunk-slot plan and workspace carve-up for the
// KDA chunked forward.  Pure C++ (no HIP calls), so every error path is testable without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>

#include "kda.h"

namespace kda {

constexpr int kChunk = 64;   // tokens per chunk (FlashKDA README, section 功能说明: 64-token chunks)
constexpr int kThreads = 256;
// Head dims: d_k = d_v = D with D = 128 (FlashKDA README, section 约束说明) or D = 64.
constexpr bool head_dim_ok(int d) { return d == 64 || d == 128; }

// Per (chunk slot, value head) workspace record for head dim D, in bytes.  Layouts are the MFMA
// fragment orders the scan kernel reads (see kda_kernels.hip).  U and K_dec (at most |k| <= 1
// with L2-normalised keys) are fp16, 11 significant bits, three more than bf16: the innovation
// V_new = U - W S^T (a small difference of large terms once the state predicts v well) is formed
// in fp32 and multiplied with K_dec on the fp16 MFMA as an fp16 hi/lo pair.
constexpr size_t rec_w_bytes(int d) { return size_t(kChunk) * d * 2; }       // W       bf16
constexpr size_t rec_q_bytes(int d) { return size_t(kChunk) * d * 2; }       // Q'      bf16
constexpr size_t rec_k_bytes(int d) { return size_t(kChunk) * d * 2; }       // K_dec   fp16
constexpr size_t rec_u_bytes(int d) { return size_t(kChunk) * d * 2; }       // U       fp16
constexpr size_t rec_o_bytes(int d) { return size_t(kChunk) * d * 2; }       // O_intra bf16
constexpr size_t rec_g_bytes(int d) { return size_t(d) * 4; }                // gamma_last fp32
constexpr size_t rec_bytes(int d) {
    return rec_w_bytes(d) + rec_q_bytes(d) + rec_k_bytes(d) + rec_u_bytes(d) + rec_o_bytes(d) +
           rec_g_bytes(d);
}
static_assert(rec_bytes(128) == 82432, "record of a 128-dim head");

struct Plan {
    int layout = 0;
    int d = 128;               // head dim (d_k = d_v)
    int batch = 0, seq_len = 0, n_qk = 0, n_v = 0, group = 0;
    int nc_max = 0;            // BNSD/BSND: chunk slots per batch row, ceil(S / 64)
    int64_t n_slots = 0;       // chunk slots: B * nc_max, or floor(T / 64) + N for TND
    int64_t n_records = 0;     // n_slots * n_v
    int64_t intra_blocks = 0;  // one workgroup per record
    int intra_hv = 1;          // waves per 16-token block of the intra kernel: 2 (eight waves,
                               // each with half the channels) when the whole grid is resident
                               // at once (<= 512 workgroups), else 1 (four waves)
    int64_t scan_blocks = 0;   // one workgroup per (sequence, value head, Dv tile), XCD padded
    int scan_nt = 1;           // 16-row Dv tiles per scan workgroup (1, 2 or 4)
    int scan_tiles = 0;        // scan workgroups per (sequence, head) = (d/16) / scan_nt
    bool scan_pf = false;      // one-level scan with a record prefetch wave (<= 256 workgroups,
                               // scan_nt <= 2)
    int seg_p = 1;             // segments per sequence of the two-level scan (1 = one level)
    int64_t seg_blocks = 0;    // two-level: segment pass, (2 seg_p - 1) d/16 per (sequence, head)
    int64_t comb_blocks = 0;   // two-level: segment combine, d/16 per (sequence, head)
    int64_t out_blocks = 0;    // two-level: output completion, one per record, then one per
                               // Dv tile of each (sequence, head) for the final state
    // byte offsets of each workspace array (256-byte aligned)
    size_t off_w = 0, off_q = 0, off_k = 0, off_u = 0, off_o = 0, off_g = 0;
    // two-level only: per (sequence, head, segment) transfer matrix P_s (transposed, fp16),
    // zero-start end state N_s (fp32) and entry state S_in(s) (bf16), d x d each; per record
    // the zero-start outputs
    // O0 and the propagated queries R = Q' P^T of the segment's chunks, 64 x d bf16 each
    size_t off_pt = 0, off_n = 0, off_sin = 0, off_o0 = 0, off_r = 0;
    size_t total = 0;
};

// Validates the shape alone; fills `plan` when it is valid.
kda_status make_plan(const kda_shape* shape, Plan* plan);

// Validates pointers and sizes of a call against a valid plan.  `gate` is the raw-gate
// activation (g then points at the raw bf16 gate) or NULL (g is the fp32 activated gate).
kda_status check_call(const kda_shape* shape, const Plan& plan, const void* q, const void* k,
                      const void* v, const void* g, const kda_raw_gate* gate, const void* beta,
                      const float* initial_state, const int32_t* cu_seqlens, const void* out,
                      const float* final_state, const void* workspace,
                      size_t workspace_bytes);

}  // namespace kda
