// kda_abi.cpp -- the extern "C" boundary declared in include/kda.h.
//
// Every argument is validated here, on the host, before the first HIP call;
// an error return has launched nothing and touched no device memory.  Then
// the matching kernel variant is picked and launched on the caller's stream.
#include <stdint.h>
#include <stdlib.h>

#include <atomic>

#include "kda.h"
#include "kda_internal.h"
#include "kda_backward.h"

namespace {

using kda::PrefillVariant;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// KDA_VALIDATE=1 turns on the device-side precondition check (read per call).
bool validate_enabled() {
    const char* env = getenv("KDA_VALIDATE");
    return env && env[0] == '1' && env[1] == '\0';
}

int default_chunk(int32_t dtype) { (void)dtype; return 16; }

int resolve_chunk(int32_t dtype, int32_t chunk) { return chunk == 0 ? default_chunk(dtype) : chunk; }

const PrefillVariant* variants(int32_t dtype, int* count) {
    if (dtype == KDA_DTYPE_BF16) return kda::prefill_variants_bf16(count);
    if (dtype == KDA_DTYPE_F32) return kda::prefill_variants_f32(count);
    *count = 0;
    return nullptr;
}

// Compute units of the current device, queried once per device.
int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

bool kind_built(int32_t dtype, int32_t D, int32_t C, int kind) {
    int count = 0;
    const PrefillVariant* tab = variants(dtype, &count);
    for (int i = 0; i < count; ++i)
        if (tab[i].D == D && tab[i].C == C && tab[i].kind == kind) return true;
    return false;
}

// Kernel kind a call runs: 3 for the backward's forward run (bf16 blocked
// checkpoints, no o), 2 for the fused gate / norm, else the plan's kernel
// (the pipeline where it is built when the plan leaves it to the library).
// -1 when the combination is not built.
int plan_kind(int32_t dtype, int32_t D, int32_t C, bool fused, bool ckb, int32_t kernel) {
    int kind;
    if (ckb) kind = 3;
    else if (fused) kind = kernel == KDA_KERNEL_CHUNK_STAGED ? -1 : 2;
    else if (kernel == KDA_KERNEL_PIPELINED) kind = 1;
    else if (kernel == KDA_KERNEL_CHUNK_STAGED) kind = 0;
    else if (kernel == KDA_KERNEL_AUTO) kind = kind_built(dtype, D, C, 1) ? 1 : 0;
    else kind = -1;
    return kind >= 0 && kind_built(dtype, D, C, kind) ? kind : -1;
}

// Value columns per workgroup, in 16-column waves.  Fewer columns per
// (sequence, head) means more workgroups (d_v slabs): that fills more compute
// units when there are few (sequence, head) recurrences, and each workgroup's
// serial chain of chunks gets shorter, but every slab repeats the d_k-side
// work (decay, Gram, solve).  The chunk-staged kernel keeps whole heads (8
// waves, fastest on MI355X for the K3 shapes at every batch size tried).  The
// pipelined kernel halves the slab while the grid still fits in one pass over
// the compute units (96 heads -> 2 slabs, 16 heads -> 8); the segment scan
// runs whole heads (its items already fill the device).  An explicit slab
// width must be built for the kernel.  Results are bitwise identical across
// slab widths.
const PrefillVariant* pick_variant(int32_t dtype, int32_t D, int32_t C, int64_t units, int kind, int32_t slab_cols,
                                   bool whole_heads) {
    int count = 0;
    const PrefillVariant* tab = variants(dtype, &count);
    int want = D / 16;
    if (slab_cols > 0) {
        if (slab_cols % 16 != 0) return nullptr;
        want = slab_cols / 16;
    } else if (kind >= 1 && !whole_heads) {
        const int64_t cus = device_cu_count();
        while (want > 1 && units * (D / (16 * want)) * 2 <= cus) want /= 2;
    }
    const PrefillVariant* best = nullptr;
    const PrefillVariant* smallest = nullptr;
    for (int i = 0; i < count; ++i) {
        const PrefillVariant& v = tab[i];
        if (v.D != D || v.C != C || v.kind != kind) continue;
        if (slab_cols > 0) {
            if (v.nwc == want) return &v;
            continue;
        }
        if (!smallest || v.nwc < smallest->nwc) smallest = &v;
        if (v.nwc <= want && (!best || v.nwc > best->nwc)) best = &v;
    }
    if (slab_cols > 0) return nullptr;
    return best ? best : smallest;
}

// Sequence-segment scan plan (kda_internal.h, PrefillParams::seg_*): G
// segments per sequence of Lc chunks each, the last one taking the rest.
// Phase 1 runs one map-pair workgroup (M and B of one segment, stage A
// shared) for each of segments 1 .. G - 2 and segment 0 with its outputs,
// phase 3 one run for each of segments 1 .. G - 1.
struct SegPlan {
    int G = 1;
    int64_t len = 0;  // tokens per segment (the last: the rest)
};

constexpr int kMaxSegments = 256;

// The library's choice: with P = compute units per (sequence, head) unit,
// G = P + 1 segments fill the device in both phases (units (G - 1)
// workgroups each), each workgroup a chain of 1 / G of the sequence (against
// the whole sequence for the direct chain), twice.  Worth it from P = 4 on,
// with segments of at least 64 chunks.
int auto_segments(int64_t units, int64_t t_seq) {
    if (units <= 0) return 1;
    const int64_t P = device_cu_count() / units;
    if (P < 4) return 1;
    const int G = (int)(P < 32 ? P + 1 : 33);
    const int64_t chunks = (t_seq + 15) / 16;
    return chunks >= 64 * (int64_t)G ? G : 1;
}

SegPlan seg_plan(int G, int64_t t_seq) {
    SegPlan sp;
    sp.G = G;
    if (G < 2) return sp;
    const int64_t chunks = (t_seq + 15) / 16;
    const int64_t lc = chunks / G;  // >= 1: plans need a chunk per segment
    sp.len = 16 * (lc < 1 ? 1 : lc);
    return sp;
}

size_t seg_workspace_bytes(int64_t units, int G, int D) {
    return G < 2 ? 0 : (size_t)units * (size_t)(G - 1) * 2 * (size_t)D * (size_t)D * sizeof(float);
}

// Segment count a call uses: 1 (direct) unless the plan asks for the scan or
// leaves it to the library, and the call is one it supports: a dense batch
// (no cu_seqlens) on the plain pipelined kernel (bf16, d = 128, chunk 16),
// without checkpoints.  0 when the plan asks for a scan the call cannot run.
int plan_segments(const kda_prefill_desc& d, bool dense, int kind) {
    const bool eligible = dense && kind == 1 && !d.fused && d.checkpoint_interval == 0 && d.num_seqs > 0 &&
                          d.total_tokens > 0 && d.d_k == 128 && d.d_v == 128;
    const int64_t units = (int64_t)d.num_seqs * d.num_heads;
    const int64_t t_seq = d.num_seqs > 0 ? d.total_tokens / d.num_seqs : 0;
    if (d.segments == 1) return 1;
    if (d.segments == 0) return eligible ? auto_segments(units, t_seq) : 1;
    if (!eligible || d.segments > kMaxSegments) return 0;
    const int64_t chunks = (t_seq + 15) / 16;
    if (chunks < d.segments) return 0;  // every segment needs a chunk
    return d.segments;
}

// Workspace a call needs; the segment scan is the only user.  kind and
// segments as the call resolves them.
size_t plan_workspace(const kda_prefill_desc& d, int segments) {
    return seg_workspace_bytes((int64_t)d.num_seqs * d.num_heads, segments, d.d_k);
}

kda_prefill_desc flat_desc(int32_t num_seqs, int64_t total_tokens, int32_t num_heads, int32_t d_k, int32_t d_v,
                           int32_t dtype, int32_t chunk_size, float scale) {
    kda_prefill_desc d;
    d.num_seqs = num_seqs;
    d.total_tokens = total_tokens;
    d.num_heads = num_heads;
    d.d_k = d_k;
    d.d_v = d_v;
    d.qkv_dtype = dtype;
    d.chunk_size = chunk_size;
    d.scale = scale;
    d.fused = 0;
    d.checkpoint_interval = 0;
    d.checkpoint_capacity = 0;
    d.kernel = KDA_KERNEL_AUTO;
    d.slab_columns = 0;
    d.segments = 0;
    return d;
}

// The kernels address 16 token rows of one chunk with 32-bit byte offsets:
// 16 rows of H heads x max(d_k, d_v) fp32 values must stay below 2^31 bytes.
bool heads_fit(int64_t num_heads, int64_t d_k, int64_t d_v) {
    return num_heads * (d_k > d_v ? d_k : d_v) * 64 <= INT32_MAX;
}

bool sizes_valid(const kda_prefill_desc& d) {
    return d.num_seqs >= 0 && d.total_tokens >= 0 && d.num_heads >= 1 && d.d_k >= 1 && d.d_v >= 1;
}

// Workspace bytes of a call described by d (dense tells whether cu_seqlens
// is absent); 0 for invalid or unsupported descriptions, which the call
// itself rejects.
size_t desc_workspace_bytes(const kda_prefill_desc& d, bool dense) {
    if (!sizes_valid(d) || d.total_tokens > INT32_MAX || !heads_fit(d.num_heads, d.d_k, d.d_v)) return 0;
    if (d.qkv_dtype != KDA_DTYPE_BF16 && d.qkv_dtype != KDA_DTYPE_F32) return 0;
    if (d.d_k != d.d_v) return 0;
    const int C = resolve_chunk(d.qkv_dtype, d.chunk_size);
    const int kind = plan_kind(d.qkv_dtype, d.d_k, C, d.fused != 0, false, d.kernel);
    if (kind < 0) return 0;
    if (dense && d.num_seqs > 0 && d.total_tokens % d.num_seqs != 0) return 0;
    const int G = plan_segments(d, dense, kind);
    return G >= 2 ? plan_workspace(d, G) : 0;
}
}  // namespace

// The output gate applied to o before it is stored (kda_prefill_output_gated).
struct GateArgs {
    const void* gate;
    const float* weight;
    float eps;
};

// dry_run: host validation only, nothing launched (the status a call with
// this workspace would return before its first HIP call).
static kda_status prefill_impl(const kda_prefill_desc& d, const kda_prefill_tensors& t, void* workspace,
                               size_t workspace_bytes, void* stream, bool dry_run = false,
                               const GateArgs* ga = nullptr) {
    const int32_t num_seqs = d.num_seqs, num_heads = d.num_heads, d_k = d.d_k, d_v = d.d_v, dtype = d.qkv_dtype;
    const int64_t total_tokens = d.total_tokens;
    const bool fused = d.fused != 0;
    const int32_t ckpt_interval = d.checkpoint_interval;
    const int64_t ckpt_capacity = d.checkpoint_capacity;
    const void *q = t.q, *k = t.k, *v = t.v, *z = t.z;
    const float *g = t.g, *beta = t.beta, *a_log = t.a_log, *initial_state = t.initial_state;
    const int32_t* cu_seqlens = t.cu_seqlens;
    void* o = t.o;
    float *final_state = t.final_state, *checkpoints = t.checkpoints;

    if (!sizes_valid(d)) return KDA_ERR_BAD_SHAPE;
    if (dtype != KDA_DTYPE_BF16 && dtype != KDA_DTYPE_F32) return KDA_ERR_UNSUPPORTED;
    if (total_tokens > INT32_MAX || !heads_fit(num_heads, d_k, d_v)) return KDA_ERR_UNSUPPORTED;
    if (num_seqs == 0 && total_tokens > 0) return KDA_ERR_BAD_SHAPE;
    if (!cu_seqlens && num_seqs > 0 && total_tokens % num_seqs != 0) return KDA_ERR_BAD_SHAPE;
    if (d.kernel < KDA_KERNEL_AUTO || d.kernel > KDA_KERNEL_CHUNK_STAGED || d.slab_columns < 0 || d.segments < 0)
        return KDA_ERR_BAD_SHAPE;
    if (!kda_prefill_supported(dtype, d_k, d_v, d.chunk_size)) return KDA_ERR_UNSUPPORTED;
    if (fused && !kda_prefill_fused_supported(dtype, d_k, d_v, d.chunk_size)) return KDA_ERR_UNSUPPORTED;
    if (total_tokens > 0 && (!q || !k || !v || !beta || !o)) return KDA_ERR_NULL_POINTER;
    if (total_tokens > 0 && !fused && !g) return KDA_ERR_NULL_POINTER;
    if (total_tokens > 0 && fused && (!z || !a_log)) return KDA_ERR_NULL_POINTER;
    if (a_log && !aligned4(a_log)) return KDA_ERR_MISALIGNED;
    const void* ptrs[] = {q, k, v, g, z, initial_state, o, final_state, workspace, checkpoints};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return KDA_ERR_MISALIGNED;
    if ((beta && !aligned4(beta)) || (cu_seqlens && !aligned4(cu_seqlens))) return KDA_ERR_MISALIGNED;
    if (o && (o == q || o == k || o == v || o == g || o == beta || o == z)) return KDA_ERR_BAD_SHAPE;
    // Checkpoints (ckpt_interval 0: none).  The interval is a positive multiple
    // of the chunk in use; the buffer holds at least floor(T_total / interval)
    // states, which bounds the sum of floor(length / interval) over sequences.
    const int C = resolve_chunk(dtype, d.chunk_size);
    if (ckpt_interval < 0 || ckpt_capacity < 0) return KDA_ERR_BAD_SHAPE;
    if (ckpt_interval > 0) {
        if (ckpt_interval % C != 0) return KDA_ERR_BAD_SHAPE;
        if (ckpt_capacity < total_tokens / ckpt_interval) return KDA_ERR_BAD_SHAPE;
        if (ckpt_capacity > 0 && !checkpoints) return KDA_ERR_NULL_POINTER;
        if ((int64_t)num_heads * d_k * d_v > INT64_MAX / (ckpt_capacity > 0 ? ckpt_capacity : 1))
            return KDA_ERR_BAD_SHAPE;
        const void* ins[] = {q, k, v, g, beta, o, initial_state, final_state};
        for (const void* ptr : ins)
            if (checkpoints && ptr == checkpoints) return KDA_ERR_BAD_SHAPE;
    }
    if (ga) {
        if (fused || ckpt_interval > 0) return KDA_ERR_UNSUPPORTED;
        if (!kda_output_gate_supported(dtype, d_v)) return KDA_ERR_UNSUPPORTED;
        if (!(ga->eps >= 0.f) || ga->eps > 1e30f) return KDA_ERR_BAD_SHAPE;  // also rejects NaN
        if (total_tokens > 0 && (!ga->gate || !ga->weight)) return KDA_ERR_NULL_POINTER;
        if ((ga->gate && !aligned16(ga->gate)) || (ga->weight && !aligned4(ga->weight))) return KDA_ERR_MISALIGNED;
        if (o && static_cast<const void*>(ga->weight) == o) return KDA_ERR_BAD_SHAPE;
        const void* ins[] = {q, k, v, g, beta};
        for (const void* ptr : ins)
            if (ga->gate && ptr == ga->gate) return KDA_ERR_BAD_SHAPE;
    }
    const int kind = plan_kind(dtype, d_k, C, fused, false, d.kernel);
    if (kind < 0) return KDA_ERR_UNSUPPORTED;
    const int G = plan_segments(d, cu_seqlens == nullptr, kind);
    if (G == 0) return KDA_ERR_UNSUPPORTED;
    const size_t need = G >= 2 ? plan_workspace(d, G) : 0;
    if (need > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;
    if (need > 0) {
        const void* io[] = {q, k, v, g, beta, initial_state, o, final_state};
        for (const void* ptr : io)
            if (ptr == workspace) return KDA_ERR_BAD_SHAPE;
    }
    if (dry_run) return KDA_OK;

    if (num_seqs == 0) return KDA_OK;
    if (total_tokens == 0 && !final_state) return KDA_OK;

    if (validate_enabled()) {
        unsigned int bad = 0;
        const int64_t n_beta = total_tokens * num_heads;
        // (the fused gate maps any z into (-5, 0): there is no g to check)
        if (kda::check_inputs(g, fused ? 0 : n_beta * d_k, beta, n_beta, cu_seqlens, num_seqs, total_tokens,
                              static_cast<hipStream_t>(stream), &bad) != hipSuccess)
            return KDA_ERR_HIP;
        if (bad) return KDA_ERR_DOMAIN;
    }

    const int64_t units = (int64_t)num_seqs * num_heads;
    const PrefillVariant* var = pick_variant(dtype, d_k, C, units, kind, d.slab_columns, G >= 2);
    if (!var) return KDA_ERR_UNSUPPORTED;
    const int nslab = d_v / (16 * var->nwc);

    kda::PrefillParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.g = g;
    p.beta = beta;
    p.S0 = initial_state;
    p.cu = cu_seqlens;
    p.o = o;
    p.Sout = final_state;
    p.T_total = total_tokens;
    p.N = num_seqs;
    p.H = num_heads;
    p.seq_len = cu_seqlens ? 0 : (int32_t)(total_tokens / num_seqs);
    p.nslab = nslab;
    p.scale = d.scale;
    p.ckpt = (ckpt_interval > 0 && total_tokens / ckpt_interval > 0) ? checkpoints : nullptr;
    p.ckpt_cap = ckpt_capacity;
    p.ckpt_interval = ckpt_interval > 0 ? ckpt_interval : 1;
    p.z = z;
    p.a_log = a_log;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (ga && G < 2 && var->launch_gate && var->nwc * 16 == d_v) {
        // whole heads in one workgroup: the gate is applied before the store
        if (kda::ws_grid_blocks(p) > INT32_MAX) return KDA_ERR_UNSUPPORTED;
        p.gate = ga->gate;
        p.gate_weight = ga->weight;
        p.gate_eps = ga->eps;
        return var->launch_gate(p, s) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }
    // otherwise o goes to the output buffer and the gate is a second pass over it
    auto gate_pass = [&]() -> kda_status {
        if (!ga || total_tokens == 0) return KDA_OK;
        kda::OutputGateParams gp;
        gp.o = o;
        gp.gate = ga->gate;
        gp.weight = ga->weight;
        gp.y = o;
        gp.rows = total_tokens * num_heads;
        gp.eps = ga->eps;
        const hipError_t e = dtype == KDA_DTYPE_BF16 ? kda::launch_output_gate_bf16(d_v, gp, device_cu_count(), s)
                                                     : kda::launch_output_gate_f32(d_v, gp, device_cu_count(), s);
        return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    };
    if (G < 2) {
        if (kda::ws_grid_blocks(p) > INT32_MAX) return KDA_ERR_UNSUPPORTED;
        if (var->launch(p, s) != hipSuccess) return KDA_ERR_HIP;
        return gate_pass();
    }
    // Segment scan: map pairs (phase 1), their chain (phase 2), runs (phase 3).
    if (!var->launch_seg || !var->launch_pair) return KDA_ERR_UNSUPPORTED;
    const SegPlan sp = seg_plan(G, p.seq_len);
    p.seg_G = sp.G;
    p.seg_len = (int32_t)sp.len;
    p.seg_ws = static_cast<float*>(workspace);
    p.seg_phase = 1;
    const int64_t b1 = kda::ws_grid_blocks(p);
    p.seg_phase = 3;
    if (b1 > INT32_MAX || kda::ws_grid_blocks(p) > INT32_MAX) return KDA_ERR_UNSUPPORTED;
    p.seg_phase = 1;
    if (var->launch_pair(p, s) != hipSuccess) return KDA_ERR_HIP;
    if (kda::launch_segment_combine(p, s) != hipSuccess) return KDA_ERR_HIP;
    p.seg_phase = 3;
    if (var->launch_seg(p, s) != hipSuccess) return KDA_ERR_HIP;
    return gate_pass();
}


extern "C" {

int32_t kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_string(int32_t s) {
    switch (s) {
        case KDA_OK: return "KDA_OK: success";
        case KDA_ERR_NULL_POINTER: return "KDA_ERR_NULL_POINTER: a required pointer is NULL";
        case KDA_ERR_BAD_SHAPE: return "KDA_ERR_BAD_SHAPE: negative or inconsistent sizes";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: no kernel built for this dtype / head dim / chunk size";
        case KDA_ERR_MISALIGNED: return "KDA_ERR_MISALIGNED: a tensor pointer is not 16-byte aligned (beta, cu_seqlens: 4-byte)";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace smaller than kda_prefill_workspace_bytes";
        case KDA_ERR_HIP: return "KDA_ERR_HIP: the HIP runtime reported an error";
        case KDA_ERR_DOMAIN: return "KDA_ERR_DOMAIN: g outside [-5, 0], beta outside [0, 1] or malformed cu_seqlens (KDA_VALIDATE=1)";
        case KDA_ERR_SCRATCH: return "KDA_ERR_SCRATCH: the call needs more workspace than the library's static buffer (kda_noalloc_scratch_bytes) holds";
        default: return "unknown kda_status";
    }
}

int32_t kda_prefill_supported(int32_t dtype, int32_t d_k, int32_t d_v, int32_t chunk_size) {
    if (d_k != d_v) return 0;
    int count = 0;
    const PrefillVariant* tab = variants(dtype, &count);
    const int C = resolve_chunk(dtype, chunk_size);
    for (int i = 0; i < count; ++i)
        if (tab[i].D == d_k && tab[i].C == C) return 1;
    return 0;
}

int32_t kda_prefill_fused_supported(int32_t dtype, int32_t d_k, int32_t d_v, int32_t chunk_size) {
    if (d_k != d_v) return 0;
    const int C = resolve_chunk(dtype, chunk_size);
    int count = 0;
    const PrefillVariant* tab = variants(dtype, &count);
    for (int i = 0; i < count; ++i)
        if (tab[i].kind == 2 && tab[i].D == d_k && tab[i].C == C) return 1;
    return 0;
}

int32_t kda_output_gate_supported(int32_t dtype, int32_t d_v) {
    return (dtype == KDA_DTYPE_BF16 || dtype == KDA_DTYPE_F32) && kda::output_gate_d_supported(d_v) ? 1 : 0;
}

kda_status kda_output_gate(int64_t total_tokens, int32_t num_heads, int32_t d_v, int32_t dtype, float eps,
                           const void* o, const void* gate, const float* weight, void* y, void* stream) {
    if (total_tokens < 0 || num_heads < 1 || d_v < 1) return KDA_ERR_BAD_SHAPE;
    if (!(eps >= 0.f) || eps > 1e30f) return KDA_ERR_BAD_SHAPE;  // also rejects NaN
    if (!kda_output_gate_supported(dtype, d_v)) return KDA_ERR_UNSUPPORTED;
    if (total_tokens > INT64_MAX / num_heads / d_v) return KDA_ERR_BAD_SHAPE;
    if (total_tokens == 0) return KDA_OK;
    if (!o || !gate || !weight || !y) return KDA_ERR_NULL_POINTER;
    if (!aligned16(o) || !aligned16(gate) || !aligned16(y) || !aligned4(weight)) return KDA_ERR_MISALIGNED;
    if (static_cast<const void*>(weight) == y) return KDA_ERR_BAD_SHAPE;
    kda::OutputGateParams p;
    p.o = o;
    p.gate = gate;
    p.weight = weight;
    p.y = y;
    p.rows = total_tokens * num_heads;
    p.eps = eps;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t err = dtype == KDA_DTYPE_BF16 ? kda::launch_output_gate_bf16(d_v, p, device_cu_count(), s)
                                                   : kda::launch_output_gate_f32(d_v, p, device_cu_count(), s);
    return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int32_t kda_decode_supported(int32_t dtype, int32_t d_k, int32_t d_v) {
    if (dtype != KDA_DTYPE_BF16 && dtype != KDA_DTYPE_F32) return 0;
    return d_k == d_v && kda::decode_d_supported(d_k) ? 1 : 0;
}

size_t kda_prefill_workspace_bytes(int32_t num_seqs, int64_t total_tokens, int32_t num_heads, int32_t d_k,
                                   int32_t d_v, int32_t dtype, int32_t chunk_size) {
    // the dense layout's need; packed batches (cu_seqlens) need none
    return desc_workspace_bytes(flat_desc(num_seqs, total_tokens, num_heads, d_k, d_v, dtype, chunk_size, 1.f), true);
}

size_t kda_prefill_ex_workspace_bytes(const kda_prefill_desc* desc) {
    return desc ? desc_workspace_bytes(*desc, true) : 0;
}

kda_status kda_prefill_ex(const kda_prefill_desc* desc, const kda_prefill_tensors* tensors, void* workspace,
                          size_t workspace_bytes, void* stream) {
    if (!desc || !tensors) return KDA_ERR_NULL_POINTER;
    return prefill_impl(*desc, *tensors, workspace, workspace_bytes, stream);
}

size_t kda_noalloc_scratch_bytes(void) { return kda::kNoallocScratchBytes; }

kda_status kda_prefill_ex_noalloc(const kda_prefill_desc* desc, const kda_prefill_tensors* tensors, void* stream) {
    if (!desc || !tensors) return KDA_ERR_NULL_POINTER;
    // The call's workspace need, from the sizes alone (host): a plan that
    // needs more than the static buffer is refused before any HIP call.
    const size_t need = desc_workspace_bytes(*desc, tensors->cu_seqlens == nullptr);
    if (need > kda::kNoallocScratchBytes) return KDA_ERR_SCRATCH;
    if (need == 0) return prefill_impl(*desc, *tensors, nullptr, 0, stream);
    // host validation first (invalid arguments report their own status)
    const kda_status pre = prefill_impl(*desc, *tensors, nullptr, 0, nullptr, true);
    if (pre == KDA_OK) return prefill_impl(*desc, *tensors, nullptr, 0, stream);
    if (pre != KDA_ERR_WORKSPACE) return pre;
    void* scratch = nullptr;
    if (kda::noalloc_scratch(&scratch) != hipSuccess) return KDA_ERR_HIP;
    return prefill_impl(*desc, *tensors, scratch, kda::kNoallocScratchBytes, stream);
}

static kda_prefill_tensors flat_tensors(const void* q, const void* k, const void* v, const float* g,
                                        const float* beta, const float* initial_state, const int32_t* cu_seqlens,
                                        void* o, float* final_state) {
    kda_prefill_tensors t;
    t.q = q;
    t.k = k;
    t.v = v;
    t.g = g;
    t.z = nullptr;
    t.a_log = nullptr;
    t.beta = beta;
    t.initial_state = initial_state;
    t.cu_seqlens = cu_seqlens;
    t.o = o;
    t.final_state = final_state;
    t.checkpoints = nullptr;
    return t;
}

kda_status kda_prefill(int32_t num_seqs, int64_t total_tokens, int32_t num_heads, int32_t d_k, int32_t d_v,
                       int32_t dtype, int32_t chunk_size, float scale, const void* q, const void* k,
                       const void* v, const float* g, const float* beta, const float* initial_state,
                       const int32_t* cu_seqlens, void* o, float* final_state, void* workspace,
                       size_t workspace_bytes, void* stream) {
    const kda_prefill_desc d = flat_desc(num_seqs, total_tokens, num_heads, d_k, d_v, dtype, chunk_size, scale);
    const kda_prefill_tensors t = flat_tensors(q, k, v, g, beta, initial_state, cu_seqlens, o, final_state);
    return prefill_impl(d, t, workspace, workspace_bytes, stream);
}

kda_status kda_prefill_output_gated(int32_t num_seqs, int64_t total_tokens, int32_t num_heads, int32_t d_k,
                                    int32_t d_v, int32_t dtype, int32_t chunk_size, float scale, const void* q,
                                    const void* k, const void* v, const float* g, const float* beta,
                                    const float* initial_state, const int32_t* cu_seqlens, const void* gate,
                                    const float* weight, float eps, void* y, float* final_state, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    const kda_prefill_desc d = flat_desc(num_seqs, total_tokens, num_heads, d_k, d_v, dtype, chunk_size, scale);
    const kda_prefill_tensors t = flat_tensors(q, k, v, g, beta, initial_state, cu_seqlens, y, final_state);
    GateArgs ga;
    ga.gate = gate;
    ga.weight = weight;
    ga.eps = eps;
    return prefill_impl(d, t, workspace, workspace_bytes, stream, false, &ga);
}

kda_status kda_prefill_fused(int32_t num_seqs, int64_t total_tokens, int32_t num_heads, int32_t d_k, int32_t d_v,
                             int32_t dtype, int32_t chunk_size, float scale, const void* q, const void* k,
                             const void* v, const void* z, const float* a_log, const float* beta,
                             const float* initial_state, const int32_t* cu_seqlens, void* o, float* final_state,
                             void* workspace, size_t workspace_bytes, void* stream) {
    kda_prefill_desc d = flat_desc(num_seqs, total_tokens, num_heads, d_k, d_v, dtype, chunk_size, scale);
    d.fused = 1;
    kda_prefill_tensors t = flat_tensors(q, k, v, nullptr, beta, initial_state, cu_seqlens, o, final_state);
    t.z = z;
    t.a_log = a_log;
    return prefill_impl(d, t, workspace, workspace_bytes, stream);
}

kda_status kda_prefill_checkpointed(int32_t num_seqs, int64_t total_tokens, int32_t num_heads, int32_t d_k,
                                    int32_t d_v, int32_t dtype, int32_t chunk_size, float scale, const void* q,
                                    const void* k, const void* v, const float* g, const float* beta,
                                    const float* initial_state, const int32_t* cu_seqlens, void* o,
                                    float* final_state, int32_t checkpoint_interval, float* checkpoints,
                                    int64_t checkpoint_capacity, void* workspace, size_t workspace_bytes,
                                    void* stream) {
    if (checkpoint_interval < 1) return KDA_ERR_BAD_SHAPE;
    kda_prefill_desc d = flat_desc(num_seqs, total_tokens, num_heads, d_k, d_v, dtype, chunk_size, scale);
    d.checkpoint_interval = checkpoint_interval;
    d.checkpoint_capacity = checkpoint_capacity;
    kda_prefill_tensors t = flat_tensors(q, k, v, g, beta, initial_state, cu_seqlens, o, final_state);
    t.checkpoints = checkpoints;
    return prefill_impl(d, t, workspace, workspace_bytes, stream);
}

// Workspace of the backward, each part at a 256-byte aligned offset: the
// state after every 16 tokens of each sequence (at most total_tokens / 16
// states per head, bf16 in the backward kernel's blocked layout), the reverse
// kernel's fp32 partials per half of the value columns, and the initial
// states in the blocked layout.
static size_t align256(size_t b) { return (b + 255) / 256 * 256; }
static size_t backward_ckpt_bytes(int64_t total_tokens, int32_t num_heads, int32_t d_k, int32_t d_v) {
    return align256((size_t)(total_tokens / 16) * (size_t)num_heads * (size_t)d_k * (size_t)d_v * 2);
}
static size_t backward_s0_bytes(int32_t num_seqs, int32_t num_heads, int32_t d_k, int32_t d_v) {
    return align256((size_t)num_seqs * (size_t)num_heads * (size_t)d_k * (size_t)d_v * 2);
}

int32_t kda_prefill_backward_supported(int32_t dtype, int32_t d_k, int32_t d_v) {
    return dtype == KDA_DTYPE_BF16 && d_k == 128 && d_v == 128 ? 1 : 0;
}

size_t kda_prefill_backward_workspace_bytes(int32_t num_seqs, int64_t total_tokens, int32_t num_heads,
                                            int32_t d_k, int32_t d_v, int32_t dtype) {
    if (!kda_prefill_backward_supported(dtype, d_k, d_v) || total_tokens < 0 || num_heads < 1 || num_seqs < 0)
        return 0;
    return backward_ckpt_bytes(total_tokens, num_heads, d_k, d_v) +
           align256(kda::backward_partial_bytes(total_tokens, num_heads)) +
           backward_s0_bytes(num_seqs, num_heads, d_k, d_v);
}

kda_status kda_prefill_backward(int32_t num_seqs, int64_t total_tokens, int32_t num_heads, int32_t d_k,
                                int32_t d_v, int32_t dtype, float scale, const void* q, const void* k,
                                const void* v, const float* g, const float* beta, const float* initial_state,
                                const int32_t* cu_seqlens, const void* d_o, const float* d_final_state, void* dq,
                                void* dk, void* dv, float* dg, float* dbeta, float* d_initial_state,
                                void* workspace, size_t workspace_bytes, void* stream) {
    if (num_seqs < 0 || total_tokens < 0 || num_heads < 1 || d_k < 1 || d_v < 1) return KDA_ERR_BAD_SHAPE;
    if (!kda_prefill_backward_supported(dtype, d_k, d_v)) return KDA_ERR_UNSUPPORTED;
    if (total_tokens > INT32_MAX || !heads_fit(num_heads, d_k, d_v)) return KDA_ERR_UNSUPPORTED;
    if (num_seqs == 0 && total_tokens > 0) return KDA_ERR_BAD_SHAPE;
    if (!cu_seqlens && num_seqs > 0 && total_tokens % num_seqs != 0) return KDA_ERR_BAD_SHAPE;
    if ((int64_t)num_seqs * num_heads > INT32_MAX) return KDA_ERR_UNSUPPORTED;
    if (total_tokens > 0 && (!q || !k || !v || !g || !beta || !d_o || !dq || !dk || !dv || !dg || !dbeta))
        return KDA_ERR_NULL_POINTER;
    const void* ptrs16[] = {q, k, v, g, d_o, initial_state, d_final_state, dq, dk, dv, dg, d_initial_state, workspace};
    for (const void* ptr : ptrs16)
        if (ptr && !aligned16(ptr)) return KDA_ERR_MISALIGNED;
    if ((beta && !aligned4(beta)) || (dbeta && !aligned4(dbeta)) || (cu_seqlens && !aligned4(cu_seqlens)))
        return KDA_ERR_MISALIGNED;
    // outputs alias neither the inputs nor each other
    const void* ins[] = {q, k, v, g, beta, initial_state, d_o, d_final_state, cu_seqlens, workspace};
    const void* outs[] = {dq, dk, dv, dg, dbeta, d_initial_state};
    for (int a = 0; a < 6; ++a) {
        if (!outs[a]) continue;
        for (const void* in : ins)
            if (outs[a] == in) return KDA_ERR_BAD_SHAPE;
        for (int b = a + 1; b < 6; ++b)
            if (outs[a] == outs[b]) return KDA_ERR_BAD_SHAPE;
    }
    const size_t need = kda_prefill_backward_workspace_bytes(num_seqs, total_tokens, num_heads, d_k, d_v, dtype);
    if (need > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;
    if (num_seqs == 0) return KDA_OK;

    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (validate_enabled()) {
        unsigned int bad = 0;
        const int64_t n_beta = total_tokens * num_heads;
        if (kda::check_inputs(g, n_beta * d_k, beta, n_beta, cu_seqlens, num_seqs, total_tokens, s, &bad) !=
            hipSuccess)
            return KDA_ERR_HIP;
        if (bad) return KDA_ERR_DOMAIN;
    }
    const int64_t units = (int64_t)num_seqs * num_heads;
    // 1. the forward pass again, for the state at every 16-token boundary (no o)
    if (total_tokens / 16 > 0) {
        const PrefillVariant* var = pick_variant(dtype, d_k, 16, units, 3, 0, false);
        if (!var) return KDA_ERR_UNSUPPORTED;
        const int nslab = d_v / (16 * var->nwc);
        if (kda::ws_pad8(units) * nslab > INT32_MAX) return KDA_ERR_UNSUPPORTED;
        kda::PrefillParams fp;
        fp.q = q;
        fp.k = k;
        fp.v = v;
        fp.g = g;
        fp.beta = beta;
        fp.S0 = initial_state;
        fp.cu = cu_seqlens;
        fp.o = nullptr;  // not read by the kind 3 kernels
        fp.Sout = nullptr;
        fp.T_total = total_tokens;
        fp.N = num_seqs;
        fp.H = num_heads;
        fp.seq_len = cu_seqlens ? 0 : (int32_t)(total_tokens / num_seqs);
        fp.nslab = nslab;
        fp.scale = scale;
        fp.ckpt = static_cast<float*>(workspace);  // bf16 blocked states (kind 3 kernels)
        fp.ckpt_cap = total_tokens / 16;
        fp.ckpt_interval = 16;
        fp.z = nullptr;
        fp.a_log = nullptr;
        if (var->launch(fp, s) != hipSuccess) return KDA_ERR_HIP;
    }
    // 2. the chunks in reverse
    kda::BackwardParams bp;
    bp.q = q;
    bp.k = k;
    bp.v = v;
    bp.g = g;
    bp.beta = beta;
    bp.S0 = initial_state;
    bp.cu = cu_seqlens;
    bp.dO = d_o;
    bp.dST = d_final_state;
    bp.ckpt = workspace;
    bp.dq = dq;
    bp.dk = dk;
    bp.dv = dv;
    bp.dg = dg;
    bp.dbeta = dbeta;
    bp.dS0 = d_initial_state;
    const size_t part_off = backward_ckpt_bytes(total_tokens, num_heads, d_k, d_v);
    bp.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + part_off);
    bp.S0b = initial_state ? static_cast<char*>(workspace) + part_off +
                                 align256(kda::backward_partial_bytes(total_tokens, num_heads))
                           : nullptr;
    bp.T_total = total_tokens;
    bp.N = num_seqs;
    bp.H = num_heads;
    bp.seq_len = cu_seqlens ? 0 : (int32_t)(total_tokens / num_seqs);
    bp.scale = scale;
    return kda::launch_backward_bf16_d128(bp, s) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_decode_step(int32_t num_seqs, int32_t num_heads, int32_t d_k, int32_t d_v, int32_t dtype,
                           float scale, const void* q, const void* k, const void* v, const float* g,
                           const float* beta, float* state, void* o, void* stream) {
    if (num_seqs < 0 || num_heads < 1 || d_k < 1 || d_v < 1) return KDA_ERR_BAD_SHAPE;
    if (!kda_decode_supported(dtype, d_k, d_v)) return KDA_ERR_UNSUPPORTED;
    if ((int64_t)num_seqs * num_heads > INT32_MAX) return KDA_ERR_UNSUPPORTED;
    if (num_seqs > 0 && (!q || !k || !v || !g || !beta || !state || !o)) return KDA_ERR_NULL_POINTER;
    const void* ptrs[] = {q, k, v, g, state, o};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return KDA_ERR_MISALIGNED;
    if (beta && !aligned4(beta)) return KDA_ERR_MISALIGNED;
    if (o && (o == q || o == k || o == v || o == g || o == beta || o == state)) return KDA_ERR_BAD_SHAPE;
    if (num_seqs == 0) return KDA_OK;
    if (validate_enabled()) {
        unsigned int bad = 0;
        const int64_t units = (int64_t)num_seqs * num_heads;
        if (kda::check_inputs(g, units * d_k, beta, units, nullptr, 0, 0, static_cast<hipStream_t>(stream), &bad) !=
            hipSuccess)
            return KDA_ERR_HIP;
        if (bad) return KDA_ERR_DOMAIN;
    }

    kda::DecodeParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.g = g;
    p.beta = beta;
    p.S = state;
    p.o = o;
    p.units = (int64_t)num_seqs * num_heads;
    p.scale = scale;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t err = dtype == KDA_DTYPE_BF16 ? kda::launch_decode_bf16(d_k, p, device_cu_count(), s)
                                                   : kda::launch_decode_f32(d_k, p, device_cu_count(), s);
    return err == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
