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
    void* o;                // [B,T,H,V] (output pass only)
    float* sT;              // [B,H,K,V] final state or null (output pass only)
    float* wsP;             // summary pass: [n_seg-1][B*H][K][K]
    float* wsL;             // summary pass: [n_seg-1][B*H][K][V]
    int B, T, H, V;
    int n_seg;              // segments of the sequence
    int cps;                // chunks per segment
    int n_vb;               // column blocks per (b, h, segment) in this launch
    int summary;            // 1: segment summary pass (no output, identity/zero start)
};

// Arguments of the segment scan: S_{j+1} = P_j S_j + L_j, written over L_j.
struct ScanParams {
    const float* s0;        // [B,H,K,V] or null
    const float* wsP;       // [n_seg-1][B*H][K][K]
    float* wsL;             // [n_seg-1][B*H][K][V], overwritten with start states
    int BH, V, n_seg;
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

// Kernel-variant selection: returns false if (dtype, K, VB) has no kernel.
bool chunk_variant_exists(int dtype, int K, int VB);

hipError_t launch_chunk(int dtype, int K, int VB, const ChunkParams& p, int grid,
                        hipStream_t stream);
hipError_t launch_scan(int K, const ScanParams& p, hipStream_t stream);
hipError_t launch_copy_state(const float* src, float* dst, size_t n, hipStream_t stream);
hipError_t launch_decode(int dtype, int K, int V, const DecodeParams& p, hipStream_t stream);

}  // namespace kda
