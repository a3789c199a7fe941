// Host-side declarations shared by the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace kda {

constexpr int kChunk = 64;       // tokens per chunk
constexpr int kSub = 16;         // tokens per sub-chunk (gate reference block)

// Arguments of one launch of the chunk kernel.
struct ChunkParams {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* beta;
    const float* s0;        // [B,H,K,V] initial state of segment 0, or null (zeros)
    const float* seg_init;  // [n_seg-1][B*H][K][V]: start state of segment s >= 1 at slot s-1
    void* o;                // [B,T,H,V] (output pass only; null: states only, no output)
    const void* gate;       // [B,T,H,V] output gate pre-activation z (o <- o sigmoid(z)), or null
    float* sT;              // [B,H,K,V] final state or null (output pass only)
    float* wsP;             // summary pass: [n_seg-1][B*H][K][K]
    float* wsL;             // summary pass: [n_seg-1][B*H][K][V]
    int B, T, H, V;
    int n_seg;              // segments of the sequence
    int cps;                // chunks per segment
    int n_vb;               // column blocks per (b, h, segment) in this launch
    int summary;            // 1: segment summary pass (no output, identity/zero start)
};

// Arguments of the fused chunk kernel (bf16, K = V = 128): one workgroup per
// (b, h, segment); four waves prepare chunk c + 1 while four carry the state
// through chunk c.  Fields as ChunkParams.
struct FusedParams {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* beta;
    const float* s0;        // [B,H,K,V] initial state of segment 0, or null (zeros)
    const float* seg_init;  // [n_seg-1][B*H][K][V]: start state of segment s >= 1 at slot s-1
    void* o;                // [B,T,H,V] (output pass)
    const void* gate;       // [B,T,H,V] output gate pre-activation z (o <- o sigmoid(z)), or null
    float* sT;              // [B,H,K,V] final state or null (output pass)
    float* wsP;             // summary pass: [n_seg-1][B*H][K][K]
    float* wsL;             // summary pass: [n_seg-1][B*H][K][V]
    int B, T, H;
    int n_seg;              // segments of the sequence
    int cps;                // chunks per segment (segments 1 ..)
    int cps0;               // chunks of segment 0 (segment s >= 1 starts at cps0 + (s - 1) cps)
    int seg_first;          // this launch's segments of each (b, h): seg_first .. seg_first + seg_count - 1
    int seg_count;
    float* seg0_L;          // output pass: segment 0's end state (slot 0 of the summaries' L), or null
    float* seg0_P;          // output pass: zeroed (slot 0 of the summaries' P), or null
};

// Arguments of the segment scan: S_{j+1} = P_j S_j + L_j, written over L_j.
struct ScanParams {
    const float* s0;        // [B,H,K,V] or null
    const float* wsP;       // [n_seg-1][B*H][K][K]
    float* wsL;             // [n_seg-1][B*H][K][V], overwritten with start states
    int BH, V, n_seg;
    // reverse scan: slot j applies the transpose of the forward transition of
    // segment n_seg - 1 - j (wsP holds the forward transitions of all n_seg
    // segments in forward order)
    int p_reverse;
};

struct DecodeParams {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* beta;
    float* state;
    void* o;
    int NH;                 // N * H
};

// T tokens per sequence in one call: q, k, g [N][T][H][K], v, o [N][T][H][V],
// beta [N][T][H]; the state is read once and written once
struct MultiDecodeParams {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* beta;
    float* state;           // [N][H][K][V], in place
    void* o;
    float* step_states;     // [N][T][H][K][V] state after each token, or null
    int N, T, H;
};

// Token-serial prefill: one workgroup per (sequence, head, 64-column block)
// walks the tokens of its chain.  Plain layout [B][T][H][*] (cu_seqlens null)
// or a packed batch [T_total][H][*] with N = B sequences at cu_seqlens.
struct TokenFwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* beta;
    const void* gate;          // output gate input [.., H, V], or null
    const float* s0;           // [B][H][K][V] or null (zeros)
    float* sT;                 // [B][H][K][V] or null; may alias s0
    void* o;
    const int* cu_seqlens;     // null: plain layout
    int B, T, H;               // T: tokens per sequence, or T_total when packed
};
hipError_t launch_token_fwd(int dtype, int K, int V, const TokenFwdParams& p, hipStream_t stream);

// ---- split path: intra-chunk pass, then state pass ----------------------------
// Per (b, h, chunk) the intra-chunk pass writes one record of the operands the
// state pass needs; all arrays row-major without padding, in the input dtype
// except egc:
//   W   [C][K]   (I + A)^{-1} diag(beta) K e^{G}
//   Qh  [C][K]   Q e^{G}
//   Mqk [C][C]   masked similarities, lower triangle incl. diagonal
//   KbT [K][C]   (K e^{G_C - G})^T
//   UtT [V][C]   ((I + A)^{-1} diag(beta) V)^T
//   egc [K]      fp32 e^{G_C}
// Records are 256-byte aligned; record (b*H + h)*NC + chunk.
struct RecLayout {
    size_t oW, oQh, oMqk, oKbT, oUtT, oEgc, bytes;
};
constexpr RecLayout rec_layout(int K, int V, int elem) {
    RecLayout r{};
    size_t o = 0;
    r.oW = o;   o += (size_t)kChunk * K * elem;
    r.oQh = o;  o += (size_t)kChunk * K * elem;
    r.oMqk = o; o += (size_t)kChunk * kChunk * elem;
    r.oKbT = o; o += (size_t)K * kChunk * elem;
    r.oUtT = o; o += (size_t)V * kChunk * elem;
    r.oEgc = o; o += (size_t)K * 4;
    r.bytes = (o + 255) & ~(size_t)255;
    return r;
}

struct IntraParams {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* beta;
    unsigned char* rec;     // [B*H*NC] records
    int B, T, H, NC;        // NC = chunks per sequence
    int n_items;            // B * H * NC
    // packed variable-length batch (B = 1, T = total tokens): null for a
    // regular batch.  Record (h * NC + global chunk); NC = chunk bound.
    const int* cu_seqlens;  // [N + 1] token offsets
    const int* chunk_off;   // [N + 1] chunk offsets (kda_varlen_prep_kernel)
    int N;
};

struct StateParams {
    const unsigned char* rec;
    const float* s0;        // [B,H,K,V] initial state of segment 0, or null (zeros)
    const float* seg_init;  // [n_seg-1][B*H][K][V]: start state of segment s >= 1 at slot s-1
    void* o;                // [B,T,H,V] (output pass only; null: states only, no output)
    const void* gate;       // [B,T,H,V] output gate pre-activation z (o <- o sigmoid(z)), or null
    float* sT;              // [B,H,K,V] final state or null (output pass only)
    float* wsP;             // summary pass: [n_seg-1][B*H][K][K]
    float* wsL;             // summary pass: [n_seg-1][B*H][K][V]
    int B, T, H, V, NC;
    int n_seg, cps, n_vb, summary;
    // packed variable-length batch (B = 1, T = total tokens; one segment):
    // null for a regular batch; workgroup (sequence, head, column block)
    const int* cu_seqlens;
    const int* chunk_off;
    int N;
    // state snapshots (output pass; null: none): after every snap_every chunks
    // that lie wholly inside sequence i, the state goes to slot
    // snap_off[i] + m of snaps [max_snaps][H][K][V] (packed batch), or to slot
    // i * snap_stride + m when snap_off is null (regular batch); slots past
    // max_snaps are skipped
    float* snaps;
    const int* snap_off;
    int snap_every, max_snaps, snap_stride;
    int snap_bf16;          // the snapshots are stored as bf16 (the backward's own copy)
    // summary pass over every segment, the last included (0: all but the last)
    int summary_all;
};

bool split_variant_exists(int dtype, int K, int V, int VB);
// offsets of a packed batch: chunk_off[i] = sum_{j<i} ceil(len_j / C), capped
// at max_chunks, and (snap_off non-null) snap_off[i] = sum_{j<i}
// floor(len_j / (snap_every C)), capped at max_snaps; lengths from cu_seqlens
// clamped to [0, T_total]
hipError_t launch_varlen_prep(const int* cu_seqlens, int N, int T_total, int max_chunks, int* chunk_off,
                              int snap_every, int max_snaps, int* snap_off, hipStream_t stream);
hipError_t launch_intra(int dtype, int K, int V, const IntraParams& p, int grid, hipStream_t stream);
hipError_t launch_state(int dtype, int K, int VB, const StateParams& p, int grid, hipStream_t stream);

// Kernel-variant selection: returns false if (dtype, K, VB) has no kernel.
bool chunk_variant_exists(int dtype, int K, int VB);
bool fused_variant_exists(int dtype, int K, int V);
hipError_t launch_fused(const FusedParams& p, int grid, hipStream_t stream);
// segment 0 with output (po, the first po.B * po.H * po.seg_count workgroups)
// beside the summaries ps, in one launch of `grid` workgroups
hipError_t launch_fused_first(const FusedParams& po, const FusedParams& ps, int grid, hipStream_t stream);

hipError_t launch_chunk(int dtype, int K, int VB, const ChunkParams& p, int grid,
                        hipStream_t stream);
hipError_t launch_scan(int K, const ScanParams& p, hipStream_t stream);
hipError_t launch_copy_state(const float* src, float* dst, size_t n, hipStream_t stream);
hipError_t launch_decode(int dtype, int K, int V, const DecodeParams& p, hipStream_t stream);

// ---- backward ------------------------------------------------------------------
struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* beta;
    const float* s0;        // [B,H,K,V] or null (zeros)
    const void* d_o;        // [B,T,H,V] dL/do or null (zeros)
    const float* dsT;       // [B,H,K,V] dL/dS_T or null (zeros)
    void* dq;               // [B,T,H,K] dtype
    void* dk;
    void* dv;               // [B,T,H,V]
    void* dg;               // [B,T,H,K]
    void* dbeta;            // [B,T,H]
    float* ds0;             // [B,H,K,V] or null
    float* ckpt;            // workspace: [B*H][ceil(T/8)][K][V] state every 8 tokens
    float* pdq;             // workspace: [V/16][B*T*H][K] partial sums per column block
    float* pdk;
    float* pda;
    float* pdb;             // [V/16][B*T*H]
    int B, T, H, V;
    // chunk-form backward (NC = chunks per sequence)
    int NC;
    const unsigned char* rec;   // [B*H*NC] records of the forward's intra-chunk pass
    const float* snaps;     // [B*NC][H][K][V]: slot b NC + c = state after chunk c
    float* adj;             // [B*H][NC][K][V]: dL/dS after chunk c (c < NC - 1)
    // bf16 copies for the fused chunk kernel (null: fp32 snaps and adj): snapshots
    // and adjoints as snaps and adj; S0 and dL/dS_T [B*H][K][V] (null: zeros)
    const void* snaps16;
    void* adj16;
    const void* s0h;
    const void* dsTh;
    // chunk-form gradients: fp32 intermediates, one slot per (b*H + h)*NC + chunk
    float* cdU;             // [C][V] dU (reverse state pass)
    float* cD;              // [C][C] tril(dO U^T)
    float* cdQh;            // [C][K] dO S^T
    float* cdKb;            // [C][K] U dS'^T
    float* cdW;             // [C][K] -dU S^T
    float* crs;             // [K] e^{G_C} rowsum(S * dS')
    float* cdKh;            // [C][K] diag(beta) dBk
    float* cEt;             // [C][C] diag(beta) E
    // reverse state pass over segments of cps chunks: the summary pass writes
    // each segment's load (wsL [K][V]) at scan slot n_seg - 1 - segment, and
    // with load_only == 0 also its transposed transition (wsP [K][K]); with
    // load_only the scan takes the transposes of the forward transitions
    // instead.  The segment scan (from dL/dS_T) leaves dL/dS after segment j
    // at wsL slot n_seg - 2 - j
    int n_seg, cps;
    float* wsP;
    float* wsL;
    int load_only;
    int n_cus;              // compute units of the device (grid of persistent kernels)
};
hipError_t launch_bwd(int dtype, int K, const BwdParams& p, hipStream_t stream);
// the reverse state pass.  summary: every segment's map (segments >= 1);
// otherwise p.adj for every chunk boundary, p.cdU for every chunk and p.ds0
// (if set), each segment from its incoming adjoint
hipError_t launch_bwd_state(bool summary, int dtype, int K, const BwdParams& p, hipStream_t stream);
// chunk-form gradients of every chunk (needs p.rec, p.snaps, p.adj, p.cdU),
// in three stages run in order: 0 value-side products, 1 Gram and back
// substitution (dv, dbeta), 2 gated products (dq, dk, dg)
bool bwd_chunk_variant_exists(int dtype, int K, int V);
hipError_t launch_bwd_chunk(int stage, int dtype, int K, int V, const BwdParams& p, hipStream_t stream);
// the three stages in one launch, one workgroup per chunk (needs p.rec,
// p.snaps, p.adj, p.cdU; no other intermediate): bf16 with K = V = 128
bool bwd_fused_variant_exists(int dtype, int K, int V);
hipError_t launch_bwd_fused(const BwdParams& p, hipStream_t stream);
// n fp32 values to bf16 (round to nearest even)
hipError_t launch_to_bf16(const float* src, void* dst, size_t n, hipStream_t stream);
size_t bwd_workspace_bytes(int B, int T, int H, int K, int V);
hipError_t launch_decode_multi(int dtype, int K, int V, const MultiDecodeParams& p, hipStream_t stream);

}  // namespace kda

#include "kda.h"

namespace kda {

// The prefill of kda_chunk_fwd_planned with at most ws_cap bytes of workspace
// at ws.  plan NULL: the library's plan when its workspace fits, else the
// single-pass plan with as many of the library's segments as fit (one segment
// needs no workspace); an explicit plan that does not fit is
// KDA_ERR_WORKSPACE.  launch false runs every host check and the plan choice
// (ws may then be null) and returns before any HIP call other than the
// device query of a plan left to the library.  Defined in kda_api.cpp.
kda_status chunk_fwd_bounded(int B, int T, int H, int K, int V, kda_dtype dt, const void* q, const void* k,
                             const void* v, const void* g, const void* beta, const float* initial_state,
                             void* o, float* final_state, const kda_plan* plan, void* ws, size_t ws_cap,
                             bool launch, hipStream_t stream);

}  // namespace kda
