// C ABI of libkda.so: argument validation, plan selection and launches.
// The declarations and their contracts are in include/kda.h.
#include "kda.h"
#include "kda_internal.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

using namespace kda;

namespace {

// ---- optional per-launch timing (kda_profile_start / kda_profile_stop) ------
// While active, every kernel launch is bracketed by two HIP events recorded on
// the launch stream.  The one piece of process-wide state of the library: off
// unless started; a mutex guards the record, so launches from several threads
// are each recorded whole (they serialise while profiling is on).
struct LaunchProfiler {
    int cap = 0, n = 0;
    hipEvent_t* ev = nullptr;          // 2 * cap events
    const char** names = nullptr;      // cap launch names
};
LaunchProfiler g_prof;
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};

template <class F>
hipError_t launch_timed(const char* name, hipStream_t st, F&& launch) {
    if (!g_prof_on.load(std::memory_order_acquire)) return launch();
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof.ev || g_prof.n >= g_prof.cap) return launch();
    const int i = g_prof.n++;
    (void)hipEventRecord(g_prof.ev[2 * i], st);
    const hipError_t e = launch();
    (void)hipEventRecord(g_prof.ev[2 * i + 1], st);
    g_prof.names[i] = name;
    return e;
}

// caller holds g_prof_mu
void profiler_release() {
    if (g_prof.ev)
        for (int i = 0; i < 2 * g_prof.cap; ++i) (void)hipEventDestroy(g_prof.ev[i]);
    delete[] g_prof.ev;
    delete[] g_prof.names;
    g_prof = LaunchProfiler{};
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_size(kda_dtype dt) { return dt == KDA_BF16 ? 2 : 4; }

kda_status check_dtype(kda_dtype dt) {
    return (dt == KDA_F32 || dt == KDA_BF16) ? KDA_OK : KDA_ERR_INVALID_ARG;
}

// Sizes the chunk kernels implement.
kda_status check_prefill_sizes(int B, int T, int H, int K, int V, kda_dtype dt) {
    if (B < 0 || T < 0 || H < 0 || K <= 0 || V <= 0) return KDA_ERR_INVALID_ARG;
    if (check_dtype(dt) != KDA_OK) return KDA_ERR_INVALID_ARG;
    if (!(K == 64 || K == 128) || !(V == 64 || V == 128)) return KDA_ERR_UNSUPPORTED;
    // every index stays within size_t and every grid within int
    const double rows = (double)B * (double)T * (double)H;
    if (rows * (double)(K > V ? K : V) > 9.0e18) return KDA_ERR_UNSUPPORTED;
    if ((double)B * H * 2.0 * 1024 > 2.0e9) return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
}

bool ranges_overlap(const void* a, const void* b, size_t n) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return n > 0 && ((x < y) ? (y < x + n) : (x < y + n));
}

bool ranges_partially_overlap(const void* a, const void* b, size_t n) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    if (x == y) return false;
    return (x < y) ? (y < x + n) : (x < y + n);
}

kda_status device_cus(int* cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return KDA_ERR_HIP;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return KDA_ERR_HIP;
    *cus = n;
    return KDA_OK;
}

// Resolve a (possibly partial) requested plan.  Needs the device CU count
// only when something is left for the library to choose (cus_fixed > 0:
// plan for that many CUs instead of querying the device).
kda_status resolve_plan(int B, int T, int H, int K, int V, kda_dtype dt, const kda_plan* req,
                        kda_plan* out, int* cps_out, int cus_fixed = 0) {
    const int n_chunks = (T + kChunk - 1) / kChunk;
    const long bh = (long)B * H;
    int vb = req ? req->v_block : 0;
    int ns = req ? req->n_seg : 0;
    int split = req ? req->split : 0;
    if (vb < 0 || ns < 0 || split < 0 || split > 4) return KDA_ERR_INVALID_ARG;
    if (vb != 0 && vb != 64 && vb != 128) return KDA_ERR_INVALID_ARG;
    // the fused form wherever it exists (bf16 with K = V = 128): one
    // workgroup per (b, h, segment) holds every value column; segments until
    // the workgroups cover the CUs, each segment keeping at least 4 chunks
    // (a request for narrower column blocks keeps the other forms)
    if (split == 0 && fused_variant_exists((int)dt, K, V) && (vb == 0 || vb == V)) split = 4;
    if (split == 4) {
        if (!fused_variant_exists((int)dt, K, V) || (vb != 0 && vb != V)) return KDA_ERR_UNSUPPORTED;
        if (ns == 0) {
            int cus = cus_fixed;
            if (cus <= 0) {
                kda_status s = device_cus(&cus);
                if (s != KDA_OK) return s;
            }
            // both passes of a segmented call run (n_seg - 1) workgroups per
            // (b, h): n_seg - 1 = the (b, h) chains that fit the CUs once
            ns = 1;
            if (bh > 0 && 2 * bh <= cus) {
                const long want = cus / bh + 1;
                const long cap = n_chunks / 4;
                ns = (int)(want < cap ? want : cap);
                if (ns < 1) ns = 1;
            }
        }
        if (n_chunks > 0 && ns > n_chunks) ns = n_chunks;
        if (ns < 1) ns = 1;
        const int cps4 = n_chunks > 0 ? (n_chunks + ns - 1) / ns : 1;
        if (n_chunks > 0) ns = (n_chunks + cps4 - 1) / cps4;   // no empty segments
        out->n_seg = ns;
        out->v_block = V;
        out->split = 4;
        if (cps_out) *cps_out = cps4;
        return KDA_OK;
    }
    // the token-serial form: the only one for sizes without chunk kernels
    // (fp32 with K or V = 128); one 64-column workgroup per (b, h, block)
    if (split == 0 && !split_variant_exists((int)dt, K, V, 64) && !chunk_variant_exists((int)dt, K, 64)) split = 3;
    if (split == 3) {
        if ((vb != 0 && vb != 64) || ns > 1) return KDA_ERR_UNSUPPORTED;
        out->n_seg = 1;
        out->v_block = 64;
        out->split = 3;
        if (cps_out) *cps_out = n_chunks > 0 ? n_chunks : 1;
        return KDA_OK;
    }
    // requests no path can serve, rejected before any device query
    if (vb != 0 && vb > V) return KDA_ERR_UNSUPPORTED;
    if (vb != 0 && ns > 1 && K % vb != 0) {
        // the summary pass carries the K transition columns in whole blocks;
        // it runs whenever the request leaves more than one segment
        const int cps_req = (n_chunks + ns - 1) / ns;
        if (n_chunks > cps_req) return KDA_ERR_UNSUPPORTED;
    }
    int cus = cus_fixed;
    if (cus <= 0 && (vb == 0 || ns == 0 || split == 0)) {
        kda_status s = device_cus(&cus);
        if (s != KDA_OK) return s;
    }
    if (split == 0) {
        // the two-pass form wherever it exists: its first pass is parallel over
        // chunks, and it measured at least as fast as the single pass on every
        // shape tried, including those whose (b, h) chains alone fill the device
        split = split_variant_exists((int)dt, K, V, 64) ? 2 : 1;
    }
    const bool vb_fixed = vb != 0;
    if (split == 2) {
        // state pass: 128 value columns per workgroup (each chunk record is
        // read once per (b, h, segment)) where the sizes allow, else 64
        if (!vb_fixed) vb = (V >= 128 && (K % 128 == 0) && split_variant_exists((int)dt, K, V, 128)) ? 128 : 64;
        if (vb > V || !split_variant_exists((int)dt, K, V, vb)) return KDA_ERR_UNSUPPORTED;
        if (ns == 0) {
            // segments until the state pass has about one workgroup per CU
            // (two for 64-column blocks), each segment keeping at least 4 chunks
            const long wgs = bh * (V / vb);
            const long slots = (vb == 128 ? 1L : 2L) * cus;
            ns = 1;
            if (wgs > 0 && wgs < slots) {
                const long want = (slots + wgs - 1) / wgs;
                const long cap = n_chunks / 4;
                ns = (int)(want < cap ? want : cap);
                if (ns < 1) ns = 1;
            }
        }
    } else {
        if (vb_fixed) {
            if (vb > V || !chunk_variant_exists((int)dt, K, vb)) return KDA_ERR_UNSUPPORTED;
        } else {
            // the widest block that still gives every CU a workgroup, else 64
            vb = 64;
            if (V >= 128 && K >= 128 && chunk_variant_exists((int)dt, K, 128) && bh * (V / 128) >= cus)
                vb = 128;
            if (!chunk_variant_exists((int)dt, K, vb)) return KDA_ERR_UNSUPPORTED;
        }
        if (ns == 0) {
            // split long sequences into segments when (b, h, column block)
            // workgroups alone leave compute units idle; each segment keeps at
            // least 8 chunks so the extra summary pass stays amortised
            const long wgs = bh * (V / vb);
            ns = 1;
            if (wgs > 0 && wgs < cus) {
                const long want = (cus + wgs - 1) / wgs;
                const long cap = n_chunks / 8;
                ns = (int)(want < cap ? want : cap);
                if (ns < 1) ns = 1;
            }
        }
    }
    if (n_chunks > 0 && ns > n_chunks) ns = n_chunks;
    if (ns < 1) ns = 1;
    int cps = n_chunks > 0 ? (n_chunks + ns - 1) / ns : 1;
    if (n_chunks > 0) ns = (n_chunks + cps - 1) / cps;   // no empty segments
    // the summary pass carries the K transition columns in whole blocks
    if (ns > 1 && K % vb != 0) {
        if (vb_fixed) return KDA_ERR_UNSUPPORTED;
        vb = 64;
    }
    out->n_seg = ns;
    out->v_block = vb;
    out->split = split;
    if (cps_out) *cps_out = cps;
    return KDA_OK;
}

size_t record_bytes(int K, int V, kda_dtype dt) {
    return rec_layout(K, V, (int)elem_size(dt)).bytes;
}

size_t segment_bytes(int B, int H, int K, int V, const kda_plan& pl) {
    if (pl.n_seg <= 1) return 0;
    const size_t bh = (size_t)B * H;
    // transitions P (K x K) and local states L (K x V) of all but the last
    // segment, plus one K x V slot per (b, h) for a redirected final state
    return ((size_t)(pl.n_seg - 1) * bh * K * (size_t)(K + V) + bh * K * V) * sizeof(float);
}

size_t workspace_bytes_for(int B, int T, int H, int K, int V, kda_dtype dt, const kda_plan& pl) {
    size_t n = segment_bytes(B, H, K, V, pl);
    if (pl.split == 2) {
        const size_t nc = (size_t)(T + kChunk - 1) / kChunk;
        n = (n + 255) & ~(size_t)255;
        n += (size_t)B * H * nc * record_bytes(K, V, dt);
    }
    return n;
}

}  // namespace

extern "C" {

const char* kda_version(void) { return "kda-mi355x 0.1.0 gfx950"; }

const char* kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_INVALID_ARG: return "invalid argument";
        case KDA_ERR_UNSUPPORTED: return "unsupported sizes or dtype";
        case KDA_ERR_WORKSPACE: return "workspace missing or too small";
        case KDA_ERR_HIP: return "HIP runtime error";
        default: break;
    }
    return "unknown status";
}

kda_status kda_chunk_fwd_plan(int B, int T, int H, int K, int V, kda_dtype dt, kda_plan* plan) {
    if (!plan) return KDA_ERR_INVALID_ARG;
    kda_status s = check_prefill_sizes(B, T, H, K, V, dt);
    if (s != KDA_OK) return s;
    return resolve_plan(B, T, H, K, V, dt, nullptr, plan, nullptr);
}

size_t kda_chunk_fwd_workspace_size(int B, int T, int H, int K, int V, kda_dtype dt) {
    return kda_chunk_fwd_planned_workspace_size(B, T, H, K, V, dt, nullptr);
}

size_t kda_chunk_fwd_planned_workspace_size(int B, int T, int H, int K, int V, kda_dtype dt,
                                            const kda_plan* plan) {
    if (check_prefill_sizes(B, T, H, K, V, dt) != KDA_OK) return (size_t)-1;
    kda_plan pl;
    if (resolve_plan(B, T, H, K, V, dt, plan, &pl, nullptr) != KDA_OK) return (size_t)-1;
    return workspace_bytes_for(B, T, H, K, V, dt, pl);
}

// dry_run: every host check (sizes, pointers, plan, workspace size with the
// workspace pointer itself not yet known), then KDA_OK before any HIP call
static kda_status chunk_impl(int B, int T, int H, int K, int V, kda_dtype dt,
                             const void* q, const void* k, const void* v,
                             const void* g, const void* beta, const void* gate,
                             const float* initial_state,
                             void* o, float* final_state,
                             const kda_plan* plan,
                             void* workspace, size_t workspace_bytes,
                             hipStream_t stream, bool dry_run = false) {
    kda_status s = check_prefill_sizes(B, T, H, K, V, dt);
    if (s != KDA_OK) return s;
    const long bh = (long)B * H;
    if (bh > 0 && T > 0) {
        if (!q || !k || !v || !g || !beta || !o) return KDA_ERR_INVALID_ARG;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(o) ||
            (reinterpret_cast<uintptr_t>(beta) % elem_size(dt)) != 0)
            return KDA_ERR_INVALID_ARG;
        if (gate && !aligned16(gate)) return KDA_ERR_INVALID_ARG;
    }
    if ((initial_state && !aligned16(initial_state)) || (final_state && !aligned16(final_state)) ||
        (workspace && !aligned16(workspace)))
        return KDA_ERR_INVALID_ARG;
    const size_t state_bytes = (size_t)bh * K * V * sizeof(float);
    if (initial_state && final_state && ranges_partially_overlap(initial_state, final_state, state_bytes))
        return KDA_ERR_INVALID_ARG;
    if (bh == 0) return KDA_OK;
    hipStream_t st = stream;

    if (T == 0) {
        if (dry_run) return KDA_OK;
        if (!final_state || final_state == initial_state) return KDA_OK;
        return launch_timed("copy_state", st, [&] {
                   return launch_copy_state(initial_state, final_state, (size_t)bh * K * V, st);
               }) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }

    kda_plan pl;
    int cps = 1;
    s = resolve_plan(B, T, H, K, V, dt, plan, &pl, &cps);
    if (s != KDA_OK) return s;
    const size_t need = workspace_bytes_for(B, T, H, K, V, dt, pl);
    if (need > 0 && ((!workspace && !dry_run) || workspace_bytes < need)) return KDA_ERR_WORKSPACE;
    if (dry_run) return KDA_OK;

    if (pl.split == 4) {
        // Segment 0 runs its output beside the other segments' summaries in
        // the first launch, and a summary chunk costs about 3.5 % less than an
        // output chunk: segment 0 is made shorter by that much (the others
        // longer), so that both roles of that launch end together.  The plan
        // (and so the workspace) keeps its number of segments; if the shift
        // would leave the last segment empty, the split stays even.
        const int n_chunks = (T + kChunk - 1) / kChunk;
        int cps0 = cps;
        if (pl.n_seg > 1) {
            const int d = (cps * 35 + 500) / 1000;
            const int c0 = cps - d;
            if (d > 0 && c0 >= 1) {
                const int rest = (n_chunks - c0 + pl.n_seg - 2) / (pl.n_seg - 1);
                if (c0 + (pl.n_seg - 2) * rest < n_chunks) {
                    cps0 = c0;
                    cps = rest;
                }
            }
        }
        FusedParams fp{};
        fp.q = q; fp.k = k; fp.v = v; fp.g = g; fp.beta = beta;
        fp.B = B; fp.T = T; fp.H = H;
        fp.n_seg = pl.n_seg;
        fp.cps = cps;
        fp.cps0 = cps0;
        fp.seg_first = 0;
        fp.seg_count = pl.n_seg;
        if (pl.n_seg == 1) {
            fp.s0 = initial_state;
            fp.o = o;
            fp.gate = gate;
            fp.sT = final_state;
            return launch_timed("fused_output", st, [&] { return launch_fused(fp, (int)bh, st); }) ==
                   hipSuccess ? KDA_OK : KDA_ERR_HIP;
        }
        float* ws = reinterpret_cast<float*>(workspace);
        float* wsP = ws;
        float* wsL = wsP + (size_t)(pl.n_seg - 1) * bh * K * K;
        float* wsFinal = wsL + (size_t)(pl.n_seg - 1) * bh * K * V;
        // pass 1: segment 0 with its output (it needs no summary: its end
        // state goes to the scan as L_0 with P_0 = 0) beside the transition P
        // and local state L of segments 1 .. n_seg - 2; (n_seg - 1) workgroups
        // per (b, h), as many as pass 3
        FusedParams f0 = fp;
        f0.s0 = initial_state;
        f0.o = o;
        f0.gate = gate;
        f0.sT = nullptr;
        f0.seg_first = 0;
        f0.seg_count = 1;
        f0.seg0_L = wsL;
        f0.seg0_P = wsP;
        FusedParams f1 = fp;
        f1.wsP = wsP;
        f1.wsL = wsL;
        f1.seg_first = 1;
        f1.seg_count = pl.n_seg - 2;
        if (launch_timed("fused_summary", st, [&] {
                return launch_fused_first(f0, f1, (int)(bh * (pl.n_seg - 1)), st);
            }) != hipSuccess)
            return KDA_ERR_HIP;
        // pass 2: segment start states (S_1 = L_0)
        ScanParams scp{};
        scp.s0 = nullptr;
        scp.wsP = wsP;
        scp.wsL = wsL;
        scp.BH = (int)bh;
        scp.V = V;
        scp.n_seg = pl.n_seg;
        if (launch_timed("segment_scan", st, [&] { return launch_scan(K, scp, st); }) != hipSuccess)
            return KDA_ERR_HIP;
        // pass 3: segments 1 .. n_seg - 1 from their true start states, with
        // output (S0 was read in pass 1, so the final state may overwrite it)
        FusedParams f3 = fp;
        f3.seg_init = wsL;
        f3.o = o;
        f3.gate = gate;
        f3.sT = final_state;
        f3.seg_first = 1;
        f3.seg_count = pl.n_seg - 1;
        (void)wsFinal;
        if (launch_timed("fused_output", st, [&] {
                return launch_fused(f3, (int)(bh * (pl.n_seg - 1)), st);
            }) != hipSuccess)
            return KDA_ERR_HIP;
        return KDA_OK;
    }
    if (pl.split == 3) {
        TokenFwdParams tp{};
        tp.q = q; tp.k = k; tp.v = v; tp.g = g; tp.beta = beta; tp.gate = gate;
        tp.s0 = initial_state;
        tp.sT = final_state;
        tp.o = o;
        tp.B = B; tp.T = T; tp.H = H;
        return launch_timed("token_fwd", st, [&] { return launch_token_fwd((int)dt, K, V, tp, st); }) == hipSuccess
                   ? KDA_OK : KDA_ERR_HIP;
    }
    if (pl.split == 2) {
        // ---- intra-chunk pass: every (b, h, chunk) record at once ----------
        const int NC = (T + kChunk - 1) / kChunk;
        const size_t seg_b = (segment_bytes(B, H, K, V, pl) + 255) & ~(size_t)255;
        unsigned char* recs = reinterpret_cast<unsigned char*>(workspace) + seg_b;
        IntraParams ip{};
        ip.q = q; ip.k = k; ip.v = v; ip.g = g; ip.beta = beta;
        ip.rec = recs;
        ip.B = B; ip.T = T; ip.H = H; ip.NC = NC;
        const long items = bh * NC;
        if (items > 2000000000L) return KDA_ERR_UNSUPPORTED;
        ip.n_items = (int)items;
        int cus = 0;
        if (device_cus(&cus) != KDA_OK) return KDA_ERR_HIP;
        const int igrid = (int)(items < cus ? items : cus);
        if (launch_timed("intra_chunk", st, [&] { return launch_intra((int)dt, K, V, ip, igrid, st); }) !=
            hipSuccess)
            return KDA_ERR_HIP;
        // ---- state pass ---------------------------------------------------------
        const int vb = pl.v_block;
        StateParams sp{};
        sp.rec = recs;
        sp.B = B; sp.T = T; sp.H = H; sp.V = V; sp.NC = NC;
        sp.n_seg = pl.n_seg;
        sp.cps = cps;
        if (pl.n_seg == 1) {
            sp.s0 = initial_state;
            sp.o = o;
            sp.gate = gate;
            sp.sT = final_state;
            sp.n_vb = V / vb;
            sp.summary = 0;
            return launch_timed("state_output", st, [&] {
                       return launch_state((int)dt, K, vb, sp, (int)(bh * (V / vb)), st);
                   }) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
        }
        float* ws = reinterpret_cast<float*>(workspace);
        float* wsP = ws;
        float* wsL = wsP + (size_t)(pl.n_seg - 1) * bh * K * K;
        float* wsFinal = wsL + (size_t)(pl.n_seg - 1) * bh * K * V;
        // K = V = 128 (bf16): one 8-wave workgroup carries the transition and
        // the load columns of a segment together and stages its records once
        const int vbs = ((int)dt == 1 && K == 128 && V == 128) ? K + V : vb;
        StateParams s1 = sp;
        s1.summary = 1;
        s1.n_vb = (K + V) / vbs;
        s1.wsP = wsP;
        s1.wsL = wsL;
        if (launch_timed("state_summary", st, [&] {
                return launch_state((int)dt, K, vbs, s1, (int)(bh * (pl.n_seg - 1) * s1.n_vb), st);
            }) != hipSuccess)
            return KDA_ERR_HIP;
        ScanParams scp{};
        scp.s0 = initial_state;
        scp.wsP = wsP;
        scp.wsL = wsL;
        scp.BH = (int)bh;
        scp.V = V;
        scp.n_seg = pl.n_seg;
        if (launch_timed("segment_scan", st, [&] { return launch_scan(K, scp, st); }) != hipSuccess)
            return KDA_ERR_HIP;
        const bool aliased = final_state && final_state == initial_state;
        StateParams s3 = sp;
        s3.summary = 0;
        s3.n_vb = V / vb;
        s3.s0 = initial_state;
        s3.seg_init = wsL;
        s3.o = o;
        s3.gate = gate;
        s3.sT = aliased ? wsFinal : final_state;
        if (launch_timed("state_output", st, [&] {
                return launch_state((int)dt, K, vb, s3, (int)(bh * pl.n_seg * s3.n_vb), st);
            }) != hipSuccess)
            return KDA_ERR_HIP;
        if (aliased && launch_timed("copy_state", st, [&] {
                return launch_copy_state(wsFinal, final_state, (size_t)bh * K * V, st);
            }) != hipSuccess)
            return KDA_ERR_HIP;
        return KDA_OK;
    }

    ChunkParams p{};
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta;
    p.B = B; p.T = T; p.H = H; p.V = V;
    p.n_seg = pl.n_seg;
    p.cps = cps;
    const int vb = pl.v_block;

    if (pl.n_seg == 1) {
        p.s0 = initial_state;
        p.o = o;
        p.gate = gate;
        p.sT = final_state;
        p.n_vb = V / vb;
        p.summary = 0;
        return launch_timed("chunk_output", st, [&] {
                   return launch_chunk((int)dt, K, vb, p, (int)(bh * (V / vb)), st);
               }) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }

    float* ws = reinterpret_cast<float*>(workspace);
    float* wsP = ws;
    float* wsL = wsP + (size_t)(pl.n_seg - 1) * bh * K * K;
    float* wsFinal = wsL + (size_t)(pl.n_seg - 1) * bh * K * V;

    // pass 1: per segment (but the last), transition P and local state L
    ChunkParams p1 = p;
    p1.summary = 1;
    p1.n_vb = (K + V) / vb;
    p1.wsP = wsP;
    p1.wsL = wsL;
    if (launch_timed("chunk_summary", st, [&] {
            return launch_chunk((int)dt, K, vb, p1, (int)(bh * (pl.n_seg - 1) * p1.n_vb), st);
        }) != hipSuccess)
        return KDA_ERR_HIP;
    // pass 2: serial combine per (b, h): segment start states, over L
    ScanParams sp{};
    sp.s0 = initial_state;
    sp.wsP = wsP;
    sp.wsL = wsL;
    sp.BH = (int)bh;
    sp.V = V;
    sp.n_seg = pl.n_seg;
    if (launch_timed("segment_scan", st, [&] { return launch_scan(K, sp, st); }) != hipSuccess)
        return KDA_ERR_HIP;
    // pass 3: every segment from its true start state, with output
    const bool aliased = final_state && final_state == initial_state;
    ChunkParams p3 = p;
    p3.summary = 0;
    p3.n_vb = V / vb;
    p3.s0 = initial_state;
    p3.seg_init = wsL;
    p3.o = o;
    p3.gate = gate;
    p3.sT = aliased ? wsFinal : final_state;
    if (launch_timed("chunk_output", st, [&] {
            return launch_chunk((int)dt, K, vb, p3, (int)(bh * pl.n_seg * p3.n_vb), st);
        }) != hipSuccess)
        return KDA_ERR_HIP;
    if (aliased && launch_timed("copy_state", st, [&] {
            return launch_copy_state(wsFinal, final_state, (size_t)bh * K * V, st);
        }) != hipSuccess)
        return KDA_ERR_HIP;
    return KDA_OK;
}

kda_status kda_chunk_fwd(int B, int T, int H, int K, int V, kda_dtype dt,
                         const void* q, const void* k, const void* v,
                         const void* g,
                         const void* beta,
                         const float* initial_state,
                         void* o,
                         float* final_state,
                         void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    return chunk_impl(B, T, H, K, V, dt, q, k, v, g, beta, nullptr, initial_state, o, final_state, nullptr,
                      workspace, workspace_bytes, stream);
}

kda_status kda_chunk_fwd_planned(int B, int T, int H, int K, int V, kda_dtype dt,
                                 const void* q, const void* k, const void* v,
                                 const void* g, const void* beta,
                                 const float* initial_state,
                                 void* o, float* final_state,
                                 const kda_plan* plan,
                                 void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
    return chunk_impl(B, T, H, K, V, dt, q, k, v, g, beta, nullptr, initial_state, o, final_state, plan,
                      workspace, workspace_bytes, stream);
}

kda_status kda_chunk_fwd_gated(int B, int T, int H, int K, int V, kda_dtype dt,
                               const void* q, const void* k, const void* v,
                               const void* g, const void* beta, const void* gate,
                               const float* initial_state,
                               void* o, float* final_state,
                               const kda_plan* plan,
                               void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    if (!gate && (long)B * H > 0 && T > 0) return KDA_ERR_INVALID_ARG;
    return chunk_impl(B, T, H, K, V, dt, q, k, v, g, beta, gate, initial_state, o, final_state, plan,
                      workspace, workspace_bytes, stream);
}

// ---- packed variable-length batch --------------------------------------------------
static size_t varlen_chunk_bound(int N, int T_total) {
    // sum_i ceil(len_i / C) <= ceil(T_total / C) + N
    return (size_t)(T_total + kChunk - 1) / kChunk + (size_t)N;
}

static kda_status check_varlen_sizes(int N, int T_total, int H, int K, int V, kda_dtype dt) {
    if (N < 0) return KDA_ERR_INVALID_ARG;
    kda_status s = check_prefill_sizes(1, T_total, H, K, V, dt);
    if (s != KDA_OK) return s;
    if ((double)H * (double)varlen_chunk_bound(N, T_total) > 2.0e9 || (double)N * H * 2.0 > 2.0e9)
        return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
}

// workspace of a packed batch: chunk offsets, snapshot offsets (each N + 1
// ints, 256-byte aligned), then the chunk records
static size_t varlen_offsets_bytes(int N) { return ((size_t)(N + 1) * sizeof(int) + 255) & ~(size_t)255; }

size_t kda_chunk_fwd_varlen_workspace_size(int N, int T_total, int H, int K, int V, kda_dtype dt) {
    if (check_varlen_sizes(N, T_total, H, K, V, dt) != KDA_OK) return (size_t)-1;
    if (!split_variant_exists((int)dt, K, V, 64)) return 0;    // token-serial form
    return 2 * varlen_offsets_bytes(N) + (size_t)H * varlen_chunk_bound(N, T_total) * record_bytes(K, V, dt);
}

static kda_status varlen_impl(int N, const int* cu_seqlens, int T_total, int H, int K, int V, kda_dtype dt,
                              const void* q, const void* k, const void* v, const void* g, const void* beta,
                              const void* gate,
                              const float* initial_state, void* o, float* final_state, int snap_interval,
                              float* snapshots, int max_snapshots, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
    kda_status s = check_varlen_sizes(N, T_total, H, K, V, dt);
    if (s != KDA_OK) return s;
    if (snap_interval < 0 || max_snapshots < 0 || snap_interval % kChunk != 0) return KDA_ERR_INVALID_ARG;
    // snapshots come from the chunk state pass: none for the token-serial form
    if (snap_interval > 0 && !split_variant_exists((int)dt, K, V, 64)) return KDA_ERR_UNSUPPORTED;
    if (snap_interval > 0 && max_snapshots > 0) {
        if (!snapshots || !aligned16(snapshots)) return KDA_ERR_INVALID_ARG;
        if ((double)max_snapshots * H * K * V > 9.0e15) return KDA_ERR_INVALID_ARG;
    }
    const long nh = (long)N * H;
    if (nh > 0 && !cu_seqlens) return KDA_ERR_INVALID_ARG;
    if (H > 0 && T_total > 0) {
        if (!q || !k || !v || !g || !beta || !o) return KDA_ERR_INVALID_ARG;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(o) ||
            (reinterpret_cast<uintptr_t>(beta) % elem_size(dt)) != 0)
            return KDA_ERR_INVALID_ARG;
        if (gate && !aligned16(gate)) return KDA_ERR_INVALID_ARG;
    }
    if ((cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)) ||
        (initial_state && !aligned16(initial_state)) || (final_state && !aligned16(final_state)) ||
        (workspace && !aligned16(workspace)))
        return KDA_ERR_INVALID_ARG;
    const size_t state_bytes = (size_t)nh * K * V * sizeof(float);
    if (initial_state && final_state && ranges_partially_overlap(initial_state, final_state, state_bytes))
        return KDA_ERR_INVALID_ARG;
    if (nh == 0) return KDA_OK;
    hipStream_t st = stream;
    if (T_total == 0) {
        if (!final_state || final_state == initial_state) return KDA_OK;
        return launch_timed("copy_state", st, [&] {
                   return launch_copy_state(initial_state, final_state, (size_t)nh * K * V, st);
               }) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }
    if (!split_variant_exists((int)dt, K, V, 64)) {
        // sizes without chunk kernels: the token-serial form, per sequence
        TokenFwdParams tp{};
        tp.q = q; tp.k = k; tp.v = v; tp.g = g; tp.beta = beta; tp.gate = gate;
        tp.s0 = initial_state;
        tp.sT = final_state;
        tp.o = o;
        tp.cu_seqlens = cu_seqlens;
        tp.B = N; tp.T = T_total; tp.H = H;
        return launch_timed("token_fwd", st, [&] { return launch_token_fwd((int)dt, K, V, tp, st); }) == hipSuccess
                   ? KDA_OK : KDA_ERR_HIP;
    }
    const size_t need = kda_chunk_fwd_varlen_workspace_size(N, T_total, H, K, V, dt);
    if (!workspace || workspace_bytes < need) return KDA_ERR_WORKSPACE;
    int cus = 0;
    if (device_cus(&cus) != KDA_OK) return KDA_ERR_HIP;

    const size_t offs = varlen_offsets_bytes(N);
    int* chunk_off = reinterpret_cast<int*>(workspace);
    int* snap_off = reinterpret_cast<int*>(reinterpret_cast<unsigned char*>(workspace) + offs);
    unsigned char* recs = reinterpret_cast<unsigned char*>(workspace) + 2 * offs;
    const int ncb = (int)varlen_chunk_bound(N, T_total);
    const bool snaps = snap_interval > 0 && max_snapshots > 0;
    const int snap_every = snap_interval / kChunk;
    if (launch_timed("varlen_prep", st, [&] {
            return launch_varlen_prep(cu_seqlens, N, T_total, ncb, chunk_off, snaps ? snap_every : 0,
                                      snaps ? max_snapshots : 0, snaps ? snap_off : nullptr, st);
        }) != hipSuccess)
        return KDA_ERR_HIP;

    IntraParams ip{};
    ip.q = q; ip.k = k; ip.v = v; ip.g = g; ip.beta = beta;
    ip.rec = recs;
    ip.B = 1; ip.T = T_total; ip.H = H; ip.NC = ncb;
    ip.n_items = H * ncb;
    ip.cu_seqlens = cu_seqlens;
    ip.chunk_off = chunk_off;
    ip.N = N;
    const int igrid = ip.n_items < cus ? ip.n_items : cus;
    if (launch_timed("intra_chunk", st, [&] { return launch_intra((int)dt, K, V, ip, igrid, st); }) != hipSuccess)
        return KDA_ERR_HIP;

    // state pass: one workgroup per (sequence, head, column block); 128-column
    // blocks when they still give every CU a workgroup
    int vb = 64;
    if (V >= 128 && split_variant_exists((int)dt, K, V, 128) && nh * (V / 128) >= cus) vb = 128;
    StateParams sp{};
    sp.rec = recs;
    sp.s0 = initial_state;
    sp.o = o;
    sp.gate = gate;
    sp.sT = final_state;
    sp.B = N; sp.T = T_total; sp.H = H; sp.V = V; sp.NC = ncb;
    sp.n_seg = 1;
    sp.cps = ncb;
    sp.n_vb = V / vb;
    sp.summary = 0;
    sp.cu_seqlens = cu_seqlens;
    sp.chunk_off = chunk_off;
    sp.N = N;
    if (snaps) {
        sp.snaps = snapshots;
        sp.snap_off = snap_off;
        sp.snap_every = snap_every;
        sp.max_snaps = max_snapshots;
    }
    return launch_timed("state_output", st, [&] {
               return launch_state((int)dt, K, vb, sp, (int)(nh * (V / vb)), st);
           }) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_chunk_fwd_varlen(int N, const int* cu_seqlens, int T_total, int H, int K, int V, kda_dtype dt,
                                const void* q, const void* k, const void* v,
                                const void* g, const void* beta,
                                const float* initial_state,
                                void* o, float* final_state,
                                void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
    return varlen_impl(N, cu_seqlens, T_total, H, K, V, dt, q, k, v, g, beta, nullptr, initial_state, o,
                       final_state, 0, nullptr, 0, workspace, workspace_bytes, stream);
}

kda_status kda_chunk_fwd_varlen_gated(int N, const int* cu_seqlens, int T_total, int H, int K, int V,
                                      kda_dtype dt, const void* q, const void* k, const void* v,
                                      const void* g, const void* beta, const void* gate,
                                      const float* initial_state, void* o, float* final_state,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!gate && (long)N * H > 0 && T_total > 0) return KDA_ERR_INVALID_ARG;
    return varlen_impl(N, cu_seqlens, T_total, H, K, V, dt, q, k, v, g, beta, gate, initial_state, o,
                       final_state, 0, nullptr, 0, workspace, workspace_bytes, stream);
}

kda_status kda_chunk_fwd_varlen_snapshots(int N, const int* cu_seqlens, int T_total, int H, int K, int V,
                                          kda_dtype dt, const void* q, const void* k, const void* v,
                                          const void* g, const void* beta, const float* initial_state,
                                          void* o, float* final_state, int snapshot_interval,
                                          float* snapshots, int max_snapshots,
                                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (snapshot_interval <= 0) return KDA_ERR_INVALID_ARG;
    return varlen_impl(N, cu_seqlens, T_total, H, K, V, dt, q, k, v, g, beta, nullptr, initial_state, o,
                       final_state, snapshot_interval, snapshots, max_snapshots, workspace, workspace_bytes,
                       stream);
}

// ---- backward -------------------------------------------------------------------------
static kda_status check_bwd_sizes(int B, int T, int H, int K, int V, kda_dtype dt) {
    if (B < 0 || T < 0 || H < 0 || K <= 0 || V <= 0) return KDA_ERR_INVALID_ARG;
    if (check_dtype(dt) != KDA_OK) return KDA_ERR_INVALID_ARG;
    if (!(K == 64 || K == 128) || !(V == 64 || V == 128)) return KDA_ERR_UNSUPPORTED;
    if ((double)B * T * H * (K > V ? K : V) * 8.0 > 9.0e15 || (double)B * H * (V / 16) > 2.0e9)
        return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
}

// Chunk-form backward (where the forward's two-pass plan exists): the
// workspace holds, 256-byte aligned in this order, the forward plan's segment
// arrays, its chunk records, the state after every chunk, dL/dS after every
// chunk, then the fp32 per-chunk intermediates of the gradient kernels.
// Elsewhere the token-level schedule: checkpoints and partial sums only.
struct BwdLayout {
    bool chunked;
    kda_plan plan;
    int cps, NC;
    size_t seg, rec, snaps, adj, inter;   // byte offsets (chunk form)
    size_t s0h, dsTh;                     // bf16 copies of S0 and dL/dS_T (fused chunk kernel)
    size_t tok;                           // byte offset of the checkpoints and partial sums (token level)
    size_t total;                         // bytes
};
// fp32 values per chunk of the chunk-form intermediates: dU, then (when the
// three stages run as separate launches) D, dQh, dKb, dW, rs, dKh, Et
static size_t bwd_inter_floats(int dt, int K, int V) {
    const size_t c = kChunk;
    if (bwd_fused_variant_exists(dt, K, V)) return c * V;
    return c * V + c * c + 4 * c * K + K + c * c;
}
static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

static kda_status bwd_layout(int B, int T, int H, int K, int V, kda_dtype dt, BwdLayout* L) {
    *L = BwdLayout{};
    L->NC = (T + kChunk - 1) / kChunk;
    if (split_variant_exists((int)dt, K, V, 64) && bwd_chunk_variant_exists((int)dt, K, V) && V % 64 == 0) {
        // the forward inside the backward is planned for the 256 CUs of an
        // MI355X, so that the workspace size does not depend on the device
        const kda_plan two_pass{0, 0, 2};
        kda_status s = resolve_plan(B, T, H, K, V, dt, &two_pass, &L->plan, &L->cps, 256);
        if (s != KDA_OK) return s;
        L->chunked = L->plan.split == 2;
    }
    if (!L->chunked) {
        // whole-sequence schedule: checkpoints and partial sums only
        L->tok = 0;
        L->total = bwd_workspace_bytes(B, T, H, K, V);
        return KDA_OK;
    }
    const size_t bh = (size_t)B * H;
    // the fused chunk kernel reads the states and adjoints as bf16 (its products
    // take bf16 operands); the three-stage form reads fp32
    const bool fused = bwd_fused_variant_exists((int)dt, K, V);
    const size_t kv = (size_t)K * V * (fused ? 2 : sizeof(float));
    size_t o = 0;
    // the forward plan's segment arrays with one more transition slot: the
    // backward's summary pass keeps the last segment's transition too, whose
    // transpose the reverse scan applies first
    L->seg = o;   o += align256(segment_bytes(B, H, K, V, L->plan) +
                                (L->plan.n_seg > 1 ? bh * K * K * sizeof(float) : 0));
    L->rec = o;   o += align256(bh * L->NC * record_bytes(K, V, dt));
    L->snaps = o; o += align256(bh * L->NC * kv);
    L->adj = o;   o += align256(bh * L->NC * kv);
    L->inter = o; o += align256(bh * L->NC * bwd_inter_floats((int)dt, K, V) * sizeof(float));
    if (fused) {
        L->s0h = o;  o += align256(bh * kv);
        L->dsTh = o; o += align256(bh * kv);
    }
    L->total = o;
    return KDA_OK;
}

size_t kda_chunk_bwd_workspace_size(int B, int T, int H, int K, int V, kda_dtype dt) {
    if (check_bwd_sizes(B, T, H, K, V, dt) != KDA_OK) return (size_t)-1;
    if ((long)B * H == 0 || T == 0) return 0;
    BwdLayout L;
    if (bwd_layout(B, T, H, K, V, dt, &L) != KDA_OK) return (size_t)-1;
    return L.total;
}

kda_status kda_chunk_bwd(int B, int T, int H, int K, int V, kda_dtype dt,
                         const void* q, const void* k, const void* v, const void* g, const void* beta,
                         const float* initial_state, const void* d_o, const float* d_final_state,
                         void* dq, void* dk, void* dv, void* dg, void* dbeta, float* d_initial_state,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
    kda_status s = check_bwd_sizes(B, T, H, K, V, dt);
    if (s != KDA_OK) return s;
    const long bh = (long)B * H;
    const uintptr_t es = elem_size(dt);
    if (bh > 0 && T > 0) {
        if (!q || !k || !v || !g || !beta || !dq || !dk || !dv || !dg || !dbeta) return KDA_ERR_INVALID_ARG;
        for (const void* t : {q, k, v, g, beta, d_o, (const void*)dq, (const void*)dk, (const void*)dv,
                              (const void*)dg, (const void*)dbeta})
            if (reinterpret_cast<uintptr_t>(t) % es != 0) return KDA_ERR_INVALID_ARG;
    }
    if ((initial_state && !aligned16(initial_state)) || (d_final_state && !aligned16(d_final_state)) ||
        (d_initial_state && !aligned16(d_initial_state)) || (workspace && !aligned16(workspace)))
        return KDA_ERR_INVALID_ARG;
    // the reverse state pass reads dL/dS_T in the same launch that writes
    // dL/dS_0: the two may not share a byte (not even as an exact alias)
    if (d_initial_state && d_final_state &&
        ranges_overlap(d_initial_state, d_final_state, (size_t)bh * K * V * sizeof(float)))
        return KDA_ERR_INVALID_ARG;
    if (bh == 0) return KDA_OK;
    hipStream_t st = stream;
    if (T == 0) {
        // no tokens: dL/dS_0 = dL/dS_T
        if (!d_initial_state) return KDA_OK;
        return launch_timed("copy_state", st, [&] {
                   return launch_copy_state(d_final_state, d_initial_state, (size_t)bh * K * V, st);
               }) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }
    BwdLayout L;
    s = bwd_layout(B, T, H, K, V, dt, &L);
    if (s != KDA_OK) return s;
    if (!workspace || workspace_bytes < L.total) return KDA_ERR_WORKSPACE;
    unsigned char* ws = reinterpret_cast<unsigned char*>(workspace);
    BwdParams p{};
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta;
    p.s0 = initial_state;
    p.d_o = d_o;
    p.dsT = d_final_state;
    p.dq = dq; p.dk = dk; p.dv = dv; p.dg = dg; p.dbeta = dbeta;
    p.ds0 = d_initial_state;
    p.B = B; p.T = T; p.H = H; p.V = V;
    if (L.chunked) {
        // the forward's records and the state after every chunk (no output)
        const int NC = L.NC;
        unsigned char* recs = ws + L.rec;
        float* snaps = reinterpret_cast<float*>(ws + L.snaps);
        IntraParams ip{};
        ip.q = q; ip.k = k; ip.v = v; ip.g = g; ip.beta = beta;
        ip.rec = recs;
        ip.B = B; ip.T = T; ip.H = H; ip.NC = NC;
        const long items = bh * NC;
        if (items > 2000000000L) return KDA_ERR_UNSUPPORTED;
        ip.n_items = (int)items;
        int cus = 0;
        if (device_cus(&cus) != KDA_OK) return KDA_ERR_HIP;
        const int igrid = (int)(items < cus ? items : cus);
        if (launch_timed("bwd_intra_chunk", st, [&] { return launch_intra((int)dt, K, V, ip, igrid, st); }) !=
            hipSuccess)
            return KDA_ERR_HIP;
        const kda_plan& pl = L.plan;
        const int vb = pl.v_block;
        StateParams sp{};
        sp.rec = recs;
        sp.B = B; sp.T = T; sp.H = H; sp.V = V; sp.NC = NC;
        sp.n_seg = pl.n_seg;
        sp.cps = L.cps;
        sp.s0 = initial_state;
        // transitions P (forward order) and loads L of every segment: the
        // reverse scan applies the transposes of the same P
        float* wsP = reinterpret_cast<float*>(ws + L.seg);
        float* wsL = wsP + (size_t)pl.n_seg * bh * K * K;
        if (pl.n_seg > 1) {
            const int vbs = ((int)dt == 1 && K == 128 && V == 128) ? K + V : vb;
            StateParams s1 = sp;
            s1.summary = 1;
            s1.summary_all = 1;
            s1.n_vb = (K + V) / vbs;
            s1.wsP = wsP;
            s1.wsL = wsL;
            if (launch_timed("bwd_state_summary", st, [&] {
                    return launch_state((int)dt, K, vbs, s1, (int)(bh * pl.n_seg * s1.n_vb), st);
                }) != hipSuccess)
                return KDA_ERR_HIP;
            ScanParams scp{};
            scp.s0 = initial_state;
            scp.wsP = wsP;
            scp.wsL = wsL;
            scp.BH = (int)bh;
            scp.V = V;
            scp.n_seg = pl.n_seg;
            if (launch_timed("bwd_segment_scan", st, [&] { return launch_scan(K, scp, st); }) != hipSuccess)
                return KDA_ERR_HIP;
            sp.seg_init = wsL;
        }
        sp.summary = 0;
        sp.n_vb = V / vb;
        // the fused chunk kernel's states and adjoints are bf16 (see bwd_layout)
        const bool fused = bwd_fused_variant_exists((int)dt, K, V);
        sp.snaps = snaps;
        sp.snap_bf16 = fused ? 1 : 0;
        sp.snap_every = 1;
        sp.max_snaps = B * NC;
        sp.snap_stride = NC;
        if (launch_timed("bwd_states", st, [&] {
                return launch_state((int)dt, K, vb, sp, (int)(bh * pl.n_seg * sp.n_vb), st);
            }) != hipSuccess)
            return KDA_ERR_HIP;
        // dL/dS at every chunk boundary (and dU of every chunk), then the
        // gradients of every chunk at once
        p.NC = NC;
        p.rec = recs;
        if (fused) {
            p.snaps16 = snaps;
            p.adj16 = ws + L.adj;
            // S0 and dL/dS_T as bf16, for the first and the last chunk
            if (initial_state) {
                p.s0h = ws + L.s0h;
                if (launch_timed("bwd_s0_bf16", st, [&] {
                        return launch_to_bf16(initial_state, ws + L.s0h, (size_t)bh * K * V, st);
                    }) != hipSuccess)
                    return KDA_ERR_HIP;
            }
            if (d_final_state) {
                p.dsTh = ws + L.dsTh;
                if (launch_timed("bwd_dsT_bf16", st, [&] {
                        return launch_to_bf16(d_final_state, ws + L.dsTh, (size_t)bh * K * V, st);
                    }) != hipSuccess)
                    return KDA_ERR_HIP;
            }
        } else {
            p.snaps = snaps;
            p.adj = reinterpret_cast<float*>(ws + L.adj);
        }
        const size_t nch = (size_t)bh * NC, c = kChunk;
        float* f = reinterpret_cast<float*>(ws + L.inter);
        p.cdU = f;  f += nch * c * V;
        if (fused) f = nullptr;                 // no other intermediate
        p.cD = f;   f += nch * c * c;
        p.cdQh = f; f += nch * c * K;
        p.cdKb = f; f += nch * c * K;
        p.cdW = f;  f += nch * c * K;
        p.crs = f;  f += nch * K;
        p.cdKh = f; f += nch * c * K;
        p.cEt = f;
        // reverse state pass over the forward plan's segments: summaries,
        // scan (reusing the forward's segment arrays), then every segment
        p.n_seg = pl.n_seg;
        p.cps = L.cps;
        p.wsP = wsP;
        p.wsL = wsL;
        p.load_only = 1;
        p.n_cus = cus;
        if (pl.n_seg > 1) {
            if (launch_timed("bwd_reverse_summary", st,
                             [&] { return launch_bwd_state(true, (int)dt, K, p, st); }) != hipSuccess)
                return KDA_ERR_HIP;
            ScanParams scp{};
            scp.s0 = d_final_state;
            scp.wsP = wsP;
            scp.wsL = wsL;
            scp.BH = (int)bh;
            scp.V = V;
            scp.n_seg = pl.n_seg;
            scp.p_reverse = 1;
            if (launch_timed("bwd_reverse_scan", st, [&] { return launch_scan(K, scp, st); }) != hipSuccess)
                return KDA_ERR_HIP;
        }
        if (launch_timed("bwd_state_reverse", st, [&] { return launch_bwd_state(false, (int)dt, K, p, st); }) !=
            hipSuccess)
            return KDA_ERR_HIP;
        if (fused)
            return launch_timed("bwd_chunk_fused", st, [&] { return launch_bwd_fused(p, st); }) == hipSuccess
                       ? KDA_OK : KDA_ERR_HIP;
        static const char* const stage_names[3] = {"bwd_value_side", "bwd_solve", "bwd_gated"};
        for (int stage = 0; stage < 3; ++stage)
            if (launch_timed(stage_names[stage], st, [&] { return launch_bwd_chunk(stage, (int)dt, K, V, p, st); }) !=
                hipSuccess)
                return KDA_ERR_HIP;
        return KDA_OK;
    }
    // token-level schedule over the whole sequence
    const size_t NG = (size_t)((T + 7) / 8);
    const size_t ck_bytes = ((size_t)bh * NG * K * V * sizeof(float) + 255) & ~(size_t)255;
    const size_t BTH = (size_t)bh * T;
    const size_t ncb = (size_t)(V / 16);
    p.ckpt = reinterpret_cast<float*>(ws + L.tok);
    p.pdq = reinterpret_cast<float*>(ws + L.tok + ck_bytes);
    p.pdk = p.pdq + ncb * BTH * K;
    p.pda = p.pdk + ncb * BTH * K;
    p.pdb = p.pda + ncb * BTH * K;
    return launch_timed("backward", st, [&] { return launch_bwd((int)dt, K, p, st); }) == hipSuccess
               ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_recurrent_steps(int N, int T, int H, int K, int V, kda_dtype dt,
                               const void* q, const void* k, const void* v,
                               const void* g, const void* beta,
                               float* state, void* o, float* step_states, hipStream_t stream) {
    if (N < 0 || T < 0 || H < 0 || K <= 0 || V <= 0) return KDA_ERR_INVALID_ARG;
    if (check_dtype(dt) != KDA_OK) return KDA_ERR_INVALID_ARG;
    if (!(K == 64 || K == 128) || !(V == 64 || V == 128)) return KDA_ERR_UNSUPPORTED;
    if ((double)N * H > 1.0e9 || (double)N * T * H * (K > V ? K : V) > 9.0e15) return KDA_ERR_UNSUPPORTED;
    const long nh = (long)N * H;
    if (nh == 0 || T == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !state || !o) return KDA_ERR_INVALID_ARG;
    if (!aligned16(state) || (step_states && !aligned16(step_states))) return KDA_ERR_INVALID_ARG;
    const uintptr_t es = elem_size(dt);
    for (const void* t : {q, k, v, g, beta, (const void*)o})
        if (reinterpret_cast<uintptr_t>(t) % es != 0) return KDA_ERR_INVALID_ARG;
    if (step_states) {
        // the two buffers may not share a byte
        const uintptr_t a0 = reinterpret_cast<uintptr_t>(state), a1 = a0 + (size_t)nh * K * V * sizeof(float);
        const uintptr_t b0 = reinterpret_cast<uintptr_t>(step_states),
                        b1 = b0 + (size_t)nh * T * K * V * sizeof(float);
        if (a0 < b1 && b0 < a1) return KDA_ERR_INVALID_ARG;
    }
    MultiDecodeParams p{};
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta;
    p.state = state;
    p.o = o;
    p.step_states = step_states;
    p.N = N; p.T = T; p.H = H;
    hipStream_t st = stream;
    return launch_timed("decode_steps", st, [&] { return launch_decode_multi((int)dt, K, V, p, st); }) ==
                   hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_recurrent_step(int N, int H, int K, int V, kda_dtype dt,
                              const void* q, const void* k, const void* v,
                              const void* g, const void* beta,
                              float* state, void* o, hipStream_t stream) {
    if (N < 0 || H < 0 || K <= 0 || V <= 0) return KDA_ERR_INVALID_ARG;
    if (check_dtype(dt) != KDA_OK) return KDA_ERR_INVALID_ARG;
    if (!(K == 64 || K == 128) || !(V == 64 || V == 128)) return KDA_ERR_UNSUPPORTED;
    if ((double)N * H > 2.0e9) return KDA_ERR_UNSUPPORTED;
    const long nh = (long)N * H;
    if (nh == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !state || !o) return KDA_ERR_INVALID_ARG;
    if (!aligned16(state)) return KDA_ERR_INVALID_ARG;
    const uintptr_t es = elem_size(dt);
    for (const void* t : {q, k, v, g, beta, (const void*)o})
        if (reinterpret_cast<uintptr_t>(t) % es != 0) return KDA_ERR_INVALID_ARG;
    DecodeParams p{};
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta;
    p.state = state;
    p.o = o;
    p.NH = (int)nh;
    hipStream_t st = stream;
    return launch_timed("decode_step", st, [&] { return launch_decode((int)dt, K, V, p, st); }) ==
                   hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_profile_start(int max_launches) {
    if (max_launches <= 0 || max_launches > (1 << 20)) return KDA_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_on.store(false, std::memory_order_release);
    profiler_release();
    LaunchProfiler p;
    p.ev = new hipEvent_t[2 * (size_t)max_launches]();
    p.names = new const char*[max_launches]();
    for (int i = 0; i < 2 * max_launches; ++i) {
        if (hipEventCreate(&p.ev[i]) != hipSuccess) {
            for (int j = 0; j < i; ++j) (void)hipEventDestroy(p.ev[j]);
            delete[] p.ev;
            delete[] p.names;
            return KDA_ERR_HIP;
        }
    }
    p.cap = max_launches;
    g_prof = p;
    g_prof_on.store(true, std::memory_order_release);
    return KDA_OK;
}

int kda_profile_stop(const char** names, float* ms, int cap) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_on.store(false, std::memory_order_release);
    if (!g_prof.ev) return -1;
    const int n = g_prof.n;
    int ret = n;
    for (int i = 0; i < n; ++i) {
        float t = 0.f;
        if (hipEventSynchronize(g_prof.ev[2 * i + 1]) != hipSuccess ||
            hipEventElapsedTime(&t, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]) != hipSuccess) {
            ret = -1;
            break;
        }
        if (i < cap) {
            if (names) names[i] = g_prof.names[i];
            if (ms) ms[i] = t;
        }
    }
    profiler_release();
    return ret;
}

}  // extern "C"

namespace kda {

// kda_chunk_fwd_planned with the workspace bounded to ws_cap bytes (see
// kda_internal.h).  launch false: checks and plan choice only.
kda_status chunk_fwd_bounded(int B, int T, int H, int K, int V, kda_dtype dt, const void* q, const void* k,
                             const void* v, const void* g, const void* beta, const float* initial_state,
                             void* o, float* final_state, const kda_plan* plan, void* ws, size_t ws_cap,
                             bool launch, hipStream_t stream) {
    // the pointer and size checks of the planned call come first
    kda_status s = chunk_impl(B, T, H, K, V, dt, q, k, v, g, beta, nullptr, initial_state, o, final_state, plan,
                              nullptr, ~(size_t)0, stream, true);
    if (s != KDA_OK) return s;
    kda_plan pl{0, 0, 0};
    if ((long)B * H > 0 && T > 0) {
        s = resolve_plan(B, T, H, K, V, dt, plan, &pl, nullptr);
        if (s != KDA_OK) return s;
        if (workspace_bytes_for(B, T, H, K, V, dt, pl) > ws_cap) {
            if (plan) return KDA_ERR_WORKSPACE;
            // the library's plan keeps records: the single pass instead, with
            // as many of its segments as the bound holds (one always fits)
            kda_plan req{0, 0, 1};
            s = resolve_plan(B, T, H, K, V, dt, &req, &pl, nullptr);
            if (s != KDA_OK) return s;
            while (pl.n_seg > 1 && workspace_bytes_for(B, T, H, K, V, dt, pl) > ws_cap) {
                req = kda_plan{pl.n_seg - 1, pl.v_block, 1};
                s = resolve_plan(B, T, H, K, V, dt, &req, &pl, nullptr);
                if (s != KDA_OK) return s;
            }
            if (workspace_bytes_for(B, T, H, K, V, dt, pl) > ws_cap) return KDA_ERR_WORKSPACE;
        }
    }
    return chunk_impl(B, T, H, K, V, dt, q, k, v, g, beta, nullptr, initial_state, o, final_state,
                      pl.split ? &pl : nullptr, ws, ws_cap, stream, !launch);
}

}  // namespace kda
