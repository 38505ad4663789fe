// kda_fwd.hip -- chunked forward of Kimi Delta Attention for MI355X (gfx950).
//
// What is computed: see include/kda.h (page "nemo_automodel.components.models.
// kimi_k3.kda_fused", package docstring).  This file holds the device code and
// the C-ABI launcher.
//
// Chunk form used by the kernels (an exact restatement of the token recurrence).
// For one chunk of c <= 64 tokens r, i with state S at its start, per key
// channel G_r = g_1 + ... + g_r (cumulative log decay inside the chunk):
//
//   A_ri = beta_r sum_c kh_rc kh_ic exp(G_rc - G_ic)   (i < r, strictly lower)
//   M_ri =        sum_c qh_rc kh_ic exp(G_rc - G_ic)   (i <= r)
//   Tb   = (I + A)^-1 Diag(beta)                       (the WY / UT factor)
//   X    = V - (kh * e^G) S
//   U    = Tb X
//   O    = scale ((qh * e^G) S + M U)
//   S   <- Diag(e^{G_c}) S + (kh * e^{G_c - G})^T U
//
// Only the last four lines depend on S; they form the sequential chain of a
// (document, head) unit.  Everything above them depends only on the chunk's
// own q, k, g, beta: call it the chunk's image (Qt, Kt, KbT, M, Tb, D).
//
// Work decomposition (three launches on the caller's stream):
//   kda_schedule_kernel  validates cu_seqlens, orders the (document, head)
//                        units longest document first and decides which long
//                        documents to split (a cost model over chunk counts);
//   kda_pre_kernel       builds the images of every chunk of the split
//                        documents in parallel (two workgroups per CU) and
//                        writes them to the workspace;
//   kda_pc_kernel        one workgroup of 8 waves per CU pulls units from a
//                        counter: waves 0-3 build (fused unit) or copy in
//                        (split unit) the image of chunk i while waves 4-7
//                        chain chunk i - 1, so a long document's sequential
//                        chain is short and a fused chunk's image is built
//                        beside the chain rather than before it.
//
// Precision: Qt, Kt and the state's MFMA copy are bf16; S stays fp32 in
// registers.  M (|M| <= 1), KbT (<= 1) and Tb are fp16, and so are X and U
// where they meet them (Tb X, M U, KbT U): fp16 carries three more mantissa
// bits than bf16, and these products dominate the error (the state update's
// rounding accumulates from chunk to chunk).  Values that would not fit fp16
// are scaled by exact powers of two (Tb per chunk, X and U per wave; almost
// never taken).
// The diagonal 16x16 blocks of A and M, and the block levels of the
// triangular solve, run on fp32 MFMA.
//
// Decay factors inside a chunk can reach exp(+-64*5.5).  A and M are therefore
// built from 16-token sub-blocks, with the decay split at G_end(b), the
// cumulative decay at the last token of the column sub-block b: the right
// factor exp(G_end(b) - G_i) is <= 1; the left factor exp(G_r - G_end(b)) is
// <= 1 for an off-diagonal pair (a > b) and at most exp(15|L|) inside a
// diagonal sub-block, where the masked upper triangle stays below
// exp(15|L|) as well (sum_c |qh_c kh_c| <= 1).  With |L| <= 5.5 nothing
// overflows fp32; off-diagonal operands are all in [0, 1] and use fp16.

#include "kda_kernels.h"
#include "kda_host_checks.h"

#include <atomic>

// the main kernel with state input / output (kda_fwd_state.hip)
namespace kda_state_tu {
hipError_t launch_main_state(dim3 grid, hipStream_t stream, const void* q, const void* k,
                             const void* v, const float* g, const float* beta, void* out,
                             void* hdr, const void* docs, const void* split, const void* images,
                             int64_t T, int H, float gate_bound);
}

namespace {

// ---------------------------------------------------------------------------
// scheduler: validate cu_seqlens, order documents longest first, and choose
// the documents whose chunks are prepared in parallel ("split" documents)
// ---------------------------------------------------------------------------
// docs[i] = (first token, length) for a fused document, (-(j + 1), length) for
// split document j; split[j] = (first token, index of its first chunk in
// pre_chunks); pre_chunks[p] = (first token, length) of split chunk p.
//
// n_exact < 0: cu is self-delimiting (it ends at its first entry equal to T)
// and empty documents are dropped.  n_exact >= 0: cu has exactly n_exact + 1
// entries, every document is listed (empty ones too: they still pass their
// state through) and doc_ids[i] receives the index of docs[i] in cu.
__global__ __launch_bounds__(SCHED_THREADS) void kda_schedule_kernel(
    const int32_t* __restrict__ cu, int T, int H, int n_cu, int cap_chunks, int policy,
    int n_exact, const float* h0, float* ht, float* chunk_states, WorkHeader* __restrict__ hdr,
    int2* __restrict__ docs, int* __restrict__ doc_ids, int2* __restrict__ split,
    int2* __restrict__ pre_chunks) {
  if (threadIdx.x == 0) {
    hdr->chunk_states = chunk_states;
    hdr->n_state_docs = n_exact >= 0 ? n_exact : 0;
    hdr->h0 = h0;
    hdr->ht = ht;
    hdr->doc_ids = doc_ids;
    hdr->status_word = &g_kda_status;
  }
  __shared__ int s_vals[SCHED_THREADS];
  __shared__ int s_term;
  __shared__ int s_bad;
  __shared__ int s_carry;
  __shared__ int s_hist[NBUCKET];
  __shared__ int s_count;
  __shared__ unsigned long long s_total;
  __shared__ int s_nsplit;
  __shared__ int s_split_chunks;
  __shared__ int s_base[MAX_SPLIT_DOCS];
  const int tid = threadIdx.x;

  int n;  // number of documents (entries 0..n of cu are valid)
  const bool keep_empty = n_exact >= 0;
  if (cu == nullptr) {
    n = 1;
  } else if (n_exact >= 0) {
    // ---- 1'. exactly n_exact + 1 entries: 0, non-decreasing, ending at T
    if (tid == 0) s_bad = 0;
    __syncthreads();
    for (int i = tid; i <= n_exact; i += SCHED_THREADS) {
      const int val = cu[i];
      bool bad = (i == 0) ? (val != 0) : (val < cu[i - 1] || val > T);
      if (i == n_exact && val != T) bad = true;
      if (bad) atomicOr(&s_bad, 1);
    }
    __syncthreads();
    n = n_exact;
  } else {
    // ---- 1. find the terminating entry (first entry equal to T) and validate
    if (tid == 0) { s_term = INT32_MAX; s_bad = 0; s_carry = 0; }
    __syncthreads();
    const int32_t* page = reinterpret_cast<const int32_t*>(reinterpret_cast<uintptr_t>(cu) & ~uintptr_t(4095));
    const int64_t first_idx = page - cu;  // index of page[0] relative to cu (<= 0)
    for (int64_t step = 0;; ++step) {
      const int64_t idx = first_idx + step * SCHED_THREADS + tid;  // entry index of this thread
      const bool mine = idx >= 0 && idx <= (int64_t)T;
      int val = 0;
      if (mine) val = page[step * SCHED_THREADS + tid];
      s_vals[tid] = val;
      __syncthreads();
      if (mine) {
        if (val == T) atomicMin(&s_term, (int)idx);
      }
      __syncthreads();
      const int term = s_term;
      if (mine && idx <= (int64_t)term) {
        int prev = (tid > 0) ? s_vals[tid - 1] : s_carry;
        bool bad = false;
        if (idx == 0) bad = (val != 0);
        else bad = (val < prev) || (val > T) || (val < 0);
        if (bad) atomicOr(&s_bad, 1);
      }
      __syncthreads();
      if (s_bad || term != INT32_MAX) break;
      // no terminator in this block: continue only if entries remain allowed
      const int64_t last_idx = first_idx + (step + 1) * SCHED_THREADS - 1;
      if (last_idx >= (int64_t)T) { if (tid == 0) s_bad = 1; __syncthreads(); break; }
      if (tid == 0) s_carry = s_vals[SCHED_THREADS - 1];
      __syncthreads();
    }
    n = s_term;
  }
  if (cu != nullptr && s_bad) {
    if (tid == 0) {
      hdr->counter = 0;
      hdr->status = 1;
      hdr->n_docs = 0;
      hdr->n_units = 0;
      hdr->n_pre_units = 0;
      hdr->n_split = 0;
      atomicOr(&g_kda_status, KDA_DEV_BAD_CU_SEQLENS);
    }
    return;
  }
  auto cu_at = [&](int i) -> int { return cu ? cu[i] : (i == 0 ? 0 : T); };

  // ---- 2. histogram of chunk counts (descending order = longest first)
  for (int b = tid; b < NBUCKET; b += SCHED_THREADS) s_hist[b] = 0;
  if (tid == 0) { s_count = 0; s_total = 0; }
  __syncthreads();
  unsigned long long my_chunks = 0;
  for (int i = tid; i < n; i += SCHED_THREADS) {
    const int a = cu_at(i), len = cu_at(i + 1) - a;
    if (len > 0 || keep_empty) {
      const int nch = (len + CH - 1) / CH;
      my_chunks += nch;
      atomicAdd(&s_hist[NBUCKET - 1 - min(nch, NBUCKET - 1)], 1);
      atomicAdd(&s_count, 1);
    }
  }
  atomicAdd(&s_total, my_chunks);
  __syncthreads();
  // exclusive prefix sum over buckets (Hillis-Steele on s_vals)
  {
    const int x = (tid < NBUCKET) ? s_hist[tid] : 0;
    s_vals[tid] = x;
    __syncthreads();
    for (int d = 1; d < SCHED_THREADS; d <<= 1) {
      const int y = (tid >= d) ? s_vals[tid - d] : 0;
      __syncthreads();
      s_vals[tid] += y;
      __syncthreads();
    }
    if (tid < NBUCKET) s_hist[tid] = s_vals[tid] - x;  // exclusive
  }
  __syncthreads();
  for (int i = tid; i < n; i += SCHED_THREADS) {
    const int a = cu_at(i), len = cu_at(i + 1) - a;
    if (len > 0 || keep_empty) {
      const int nch = (len + CH - 1) / CH;
      const int pos = atomicAdd(&s_hist[NBUCKET - 1 - min(nch, NBUCKET - 1)], 1);
      docs[pos] = make_int2(a, len);
      if (keep_empty) doc_ids[pos] = i;
    }
  }
  __threadfence_block();
  __syncthreads();

  // ---- 3. split decision over the longest MAX_SPLIT_DOCS documents, staged
  // in LDS (starts in s_hist, lengths in s_vals).  Documents of 1024+ chunks
  // share the top bucket in arbitrary order; the decision only needs the list
  // to be roughly sorted.
  const int n_cand = min(s_count, MAX_SPLIT_DOCS);
  for (int i = tid; i < n_cand; i += SCHED_THREADS) {
    const int2 d = docs[i];
    s_hist[i] = d.x;
    s_vals[i] = d.y;
  }
  __syncthreads();
  if (tid == 0) {
    // estimates in float: only their order matters
    const int nd = s_count;
    const float per_cu = (float)H / (float)max(n_cu, 1);
    const float total = (float)s_total;
    auto nch_of = [&](int i) -> int { return (s_vals[i] + CH - 1) / CH; };
    int best_s = 0;
    int best_sum = 0;
    if (policy != SPLIT_NEVER && nd > 0) {
      float best = fmaxf((float)nch_of(0) * COST_FUSED, total * per_cu * COST_FUSED);
      int sum = 0, longest_split = 0;
      for (int s = 1; s <= n_cand; ++s) {
        const int c = nch_of(s - 1);
        if (c < MIN_SPLIT_CHUNKS || sum + c > cap_chunks) break;
        sum += c;
        longest_split = max(longest_split, c);
        const float pre = ceilf((float)sum * per_cu) * COST_PRE;
        // longest fused document (beyond the candidates: at most the last one's length)
        const float rest = (s < nd) ? (float)nch_of(min(s, n_cand - 1)) * COST_FUSED : 0.f;
        const float avg = ((float)sum * COST_CHAIN + (total - (float)sum) * COST_FUSED) * per_cu;
        const float bound = fmaxf((float)longest_split * COST_CHAIN, avg);
        const float est = pre + fmaxf(bound, rest);
        if (policy == SPLIT_ALWAYS || est < best) { best = est; best_s = s; best_sum = sum; }
        // once the longest document left fused is no longer the bound, more
        // splits only add prepare work (COST_PRE exceeds what a split saves,
        // COST_FUSED - COST_CHAIN): stop
        if (policy != SPLIT_ALWAYS && rest <= bound) break;
      }
    }
    // first chunk of each split document in pre_chunks (exclusive prefix sum)
    int base = 0;
    for (int j = 0; j < best_s; ++j) {
      s_base[j] = base;
      base += (int)nch_of(j);
    }
    s_nsplit = best_s;
    s_split_chunks = best_sum;
  }
  __syncthreads();
  const int ns = s_nsplit;
  for (int j = tid; j < ns; j += SCHED_THREADS) {
    split[j] = make_int2(s_hist[j], s_base[j]);
    docs[j] = make_int2(-(j + 1), s_vals[j]);
  }
  for (int j = 0; j < ns; ++j) {
    const int start = s_hist[j], len = s_vals[j], b = s_base[j];
    const int nch = (len + CH - 1) / CH;
    for (int c = tid; c < nch; c += SCHED_THREADS)
      pre_chunks[b + c] = make_int2(start + CH * c, min(CH, len - CH * c));
  }
  if (tid == 0) {
    hdr->counter = 0;
    hdr->status = 0;
    hdr->n_docs = s_count;
    hdr->n_units = s_count * H;
    hdr->n_pre_units = s_split_chunks * H;
    hdr->n_split = ns;
  }
}

// ---------------------------------------------------------------------------
// pre kernel: the state-independent part of every chunk of the split
// documents, in parallel (two workgroups per CU), written out as images
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(NTHR, 2) void kda_pre_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const float* __restrict__ g,
    const float* __restrict__ beta, WorkHeader* __restrict__ hdr,
    const int2* __restrict__ pre_chunks, uint8_t* __restrict__ images, int H, float gate_bound) {
  __shared__ PreSmem sm;
  const Lane ln = make_lane();
  if (hdr->status != 0) return;
  const int n_units = hdr->n_pre_units;
  if (n_units == 0) return;
  const Offsets of = make_offsets(H, ln.tok, ln.cg, ln.w, ln.l);
  if (ln.tid == 0) sm.gate_bad = 0;
  // every unit costs the same: workgroup b takes units b, b + grid, ...
  // The next unit's raw inputs arrive during the current one's prepare, in
  // three parts (after B0, after the tiles, after B3), into the registers the
  // prologue has consumed by then.
  auto src_of = [&](int u) {
    const int2 ch = pre_chunks[u / H];
    return raw_src(q, k, g, beta, ch.x, ch.y, H, u % H);
  };
  RawChunk cur;
  if ((int)blockIdx.x < n_units) load_raw(cur, src_of(blockIdx.x), of);
  for (int unit = blockIdx.x; unit < n_units; unit += gridDim.x) {
    const int2 ch = pre_chunks[unit / H];
    const int h = unit % H;
    const int next = unit + (int)gridDim.x;
    // the lane coordinates from a value the compiler cannot see through, so
    // that what it derives from them is not hoisted out of the loop (where it
    // would hold registers for the whole kernel)
    int t = ln.tid;
    asm volatile("" : "+v"(t));
    const Lane lnI = make_lane(t);
    const Offsets ofI = make_offsets(H, lnI.tok, lnI.cg, lnI.w, lnI.l);
    uint8_t* img = images + ((size_t)(unit / H) * H + h) * IMG_BYTES;
    const GlobalSink sink{make_rsrc(img, IMG_BYTES)};
    prepare_chunk(sm, sink, cur, ch.y, gate_bound, lnI, [&](int part) {
      if (part >= 1 && part <= 3 && next < n_units) load_raw_part(cur, src_of(next), ofI, part - 1);
    });
    // KbT and M: padded LDS staging rows -> image pieces
    const uint8_t* st = reinterpret_cast<const uint8_t*>(&sm.KbT[0][0]);
#pragma unroll
    for (int i = 0; i < IMG_KB / NTHR; ++i) {
      const int pc = lnI.tid + NTHR * i;
      bstore(*reinterpret_cast<const u32x4*>(st + (pc >> 3) * ROW_CC + (pc & 7) * 16), sink.r,
             16 * (GP_KB + pc));
    }
    const uint8_t* sm_m = st + DK * ROW_CC;
#pragma unroll
    for (int i = 0; i < (CH * (CH / 8) + NTHR - 1) / NTHR; ++i) {
      const int pc = lnI.tid + NTHR * i, row = pc >> 3, cp = pc & 7;
      const int gp = img_mt_piece(0, row, cp);
      if (gp >= 0) bstore(*reinterpret_cast<const u32x4*>(sm_m + row * ROW_CC + cp * 16), sink.r, 16 * gp);
    }
    __syncthreads();  // the staging is read out before the next unit rewrites it
  }
  __syncthreads();
  if (ln.tid == 0 && sm.gate_bad) atomicOr(&g_kda_status, KDA_DEV_GATE_RANGE);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
thread_local std::string t_last_error;

int fail(int code, const std::string& msg) {
  t_last_error = msg;
  return code;
}

// Workspaces come from a memory pool the library owns, one per device (the
// device's default pool and its attributes are left alone).  The pool keeps
// up to KDA_POOL_KEEP_BYTES reserved between calls, so that a steady stream
// of calls does not map and unmap its workspace every time; memory beyond
// that goes back to the device when the stream synchronises.
constexpr uint64_t KDA_POOL_KEEP_BYTES = uint64_t(8) << 30;

// The workspace of kda_chunk_fwd_noalloc, for callers that cannot allocate:
// one fixed array per device, kept until the process ends.  Host code never
// passes this name to a kernel (on the host it is only a stand-in for the
// symbol): it looks up each device's own address with hipGetSymbolAddress,
// once per device, and passes that.  Every call on a device shares that
// device's array, so calls that overlap on one device race; the array keeps
// the last call's contents, and the scheduler rewrites every field a call
// reads before any kernel of the call reads it.
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

struct DeviceInfo {
  int num_cu = 0;
  hipMemPool_t pool = nullptr;
  int* status_word = nullptr;  // device address of this device's g_kda_status
  uint8_t* scratch = nullptr;  // device address of this device's scratch array
};
std::mutex g_mu;
std::vector<DeviceInfo> g_devices;

// CU count, status word and scratch address of device dev (the current
// device); with_pool also creates the library's memory pool of the device.
int device_info(int dev, DeviceInfo** out, bool with_pool = true) {
  std::lock_guard<std::mutex> lock(g_mu);
  if ((int)g_devices.size() <= dev) g_devices.resize(dev + 1);
  DeviceInfo& d = g_devices[dev];
  if (d.num_cu == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return -1;
    d.num_cu = n;
  }
  if (d.scratch == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return -1;
    d.scratch = static_cast<uint8_t*>(p);
  }
  if (with_pool && d.pool == nullptr) {
    hipMemPoolProps props;
    memset(&props, 0, sizeof(props));
    props.allocType = hipMemAllocationTypePinned;
    props.handleTypes = hipMemHandleTypeNone;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool = nullptr;
    if (hipMemPoolCreate(&pool, &props) != hipSuccess || pool == nullptr) return -1;
    uint64_t keep = KDA_POOL_KEEP_BYTES;
    if (hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep) != hipSuccess) {
      (void)hipMemPoolDestroy(pool);
      return -1;
    }
    d.pool = pool;
  }
  if (d.status_word == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_kda_status)) != hipSuccess || p == nullptr) return -1;
    d.status_word = static_cast<int*>(p);
  }
  *out = &d;
  return 0;
}


// Upper bound of the chunk images of split documents in the workspace.
constexpr size_t IMAGE_BUDGET_BYTES = size_t(16) << 30;

// The choice of split documents: automatic unless a test forces it through
// kda_debug_set_split_policy (both forced settings give bit-identical results).
std::atomic<int> g_split_policy{SPLIT_AUTO};
int split_policy() { return g_split_policy.load(std::memory_order_relaxed); }

// One call of either entry point, after its argument checks.
struct Call {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const int32_t* cu;
  int64_t T;
  int H;
  float gate_bound;
  void* out;
  int n_exact;  // < 0: self-delimiting cu_seqlens; else its document count
  const float* h0;
  float* ht;
  hipStream_t stream;
  float* chunk_states = nullptr;  // S at every chunk start (the backward's forward pass)
  bool no_alloc = false;          // use the device's scratch array, allocate nothing
};

int launch(const Call& c) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(KDA_ERR_HIP, "hipGetDevice failed");
  DeviceInfo* di = nullptr;
  if (device_info(dev, &di, !c.no_alloc) != 0)
    return fail(KDA_ERR_HIP, "device query (CU count, status word, scratch) failed");
  const int64_t T = c.T;
  const int H = c.H;

  // workspace: header | docs[n_list] | doc_ids[n_list] | split[max_split] |
  // pre_chunks[cap] | images[cap][H]
  const int policy = split_policy();
  kda_check::FwdLayout lay;
  if (!kda_check::fwd_layout(T, H, c.n_exact, policy != SPLIT_NEVER, IMG_BYTES, IMAGE_BUDGET_BYTES,
                             MIN_SPLIT_CHUNKS, MAX_SPLIT_DOCS, &lay))
    return fail(KDA_ERR_BAD_SHAPE, "workspace size overflows");
  if (c.no_alloc && lay.bytes > NOALLOC_SCRATCH_BYTES) {
    // the images of split documents get what the scratch has left
    kda_check::FwdLayout base;
    if (!kda_check::fwd_layout(T, H, c.n_exact, false, IMG_BYTES, 0, MIN_SPLIT_CHUNKS,
                               MAX_SPLIT_DOCS, &base))
      return fail(KDA_ERR_BAD_SHAPE, "workspace size overflows");
    const size_t room = base.bytes <= NOALLOC_SCRATCH_BYTES ? NOALLOC_SCRATCH_BYTES - base.bytes : 0;
    if (base.bytes > NOALLOC_SCRATCH_BYTES ||
        !kda_check::fwd_layout(T, H, c.n_exact, policy != SPLIT_NEVER, IMG_BYTES, room,
                               MIN_SPLIT_CHUNKS, MAX_SPLIT_DOCS, &lay) ||
        lay.bytes > NOALLOC_SCRATCH_BYTES)
      return fail(KDA_ERR_BAD_SHAPE, "T is too large for the 64 MiB scratch of kda_chunk_fwd_noalloc "
                                     "(it needs 8 bytes per token and a few KiB)");
  }
  const size_t cap_chunks = lay.cap_chunks;
  const size_t ws_bytes = lay.bytes;
  uint8_t* ws = nullptr;
  if (c.no_alloc) {
    ws = di->scratch;
  } else if (hipMallocFromPoolAsync(reinterpret_cast<void**>(&ws), ws_bytes, di->pool, c.stream) != hipSuccess ||
             !ws) {
    return fail(KDA_ERR_ALLOC, "stream-ordered allocation of the workspace failed");
  }
  WorkHeader* hdr = reinterpret_cast<WorkHeader*>(ws);
  int2* docs = reinterpret_cast<int2*>(ws + lay.off_docs);
  int* doc_ids = c.n_exact >= 0 ? reinterpret_cast<int*>(ws + lay.off_ids) : nullptr;
  int2* split = reinterpret_cast<int2*>(ws + lay.off_split);
  int2* pre_chunks = reinterpret_cast<int2*>(ws + lay.off_pre);
  uint8_t* images = ws + lay.off_img;

  hipLaunchKernelGGL(kda_schedule_kernel, dim3(1), dim3(SCHED_THREADS), 0, c.stream, c.cu,
                     (int)T, H, di->num_cu, (int)cap_chunks, policy, c.n_exact, c.h0, c.ht,
                     c.chunk_states, hdr, docs, doc_ids, split, pre_chunks);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && cap_chunks > 0) {
    hipLaunchKernelGGL(kda_pre_kernel, dim3(2 * di->num_cu), dim3(NTHR), 0, c.stream,
                       static_cast<const bf16*>(c.q), static_cast<const bf16*>(c.k), c.g, c.beta,
                       hdr, pre_chunks, images, H, c.gate_bound);
    e = hipGetLastError();
  }
  if (e == hipSuccess) {
    if (c.h0 || c.ht || c.chunk_states) {
      e = kda_state_tu::launch_main_state(dim3(di->num_cu), c.stream, c.q, c.k, c.v, c.g, c.beta,
                                          c.out, hdr, docs, split, images, T, H, c.gate_bound);
    } else {
      hipLaunchKernelGGL(kda_pc_kernel<false>, dim3(di->num_cu), dim3(NPC), 0, c.stream,
                         static_cast<const bf16*>(c.q), static_cast<const bf16*>(c.k),
                         static_cast<const bf16*>(c.v), c.g, c.beta, static_cast<bf16*>(c.out),
                         hdr, docs, split, images, T, H, c.gate_bound);
      e = hipGetLastError();
    }
  }
  const hipError_t ef = c.no_alloc ? hipSuccess : hipFreeAsync(ws, c.stream);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  if (ef != hipSuccess) return fail(KDA_ERR_HIP, "hipFreeAsync of the workspace failed");
  return KDA_OK;
}

}  // namespace

// host helpers shared with the other translation units of the library
namespace kda_host {
int fail(int code, const std::string& msg) { return ::fail(code, msg); }
// The stateful forward with S stored at every chunk start (see
// WorkHeader::chunk_states): the first pass of the backward.  Arguments were
// checked by the caller.
int forward_with_chunk_states(const void* q, const void* k, const void* v, const float* g,
                              const float* beta, const int32_t* cu, int32_t n_docs, int64_t T,
                              int32_t H, float gate_bound, const float* h0, void* out,
                              float* chunk_states, hipStream_t stream) {
  Call c{q, k, v, g, beta, cu, T, H, gate_bound, out, n_docs, h0, nullptr, stream};
  c.chunk_states = chunk_states;
  return launch(c);
}
int device(int* num_cu, int** status_word) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  DeviceInfo* di = nullptr;
  if (device_info(dev, &di) != 0) return -1;
  *num_cu = di->num_cu;
  *status_word = di->status_word;
  return 0;
}
// stream-ordered workspace from the library's pool of the current device
hipError_t alloc_async(void** p, size_t bytes, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  DeviceInfo* di = nullptr;
  if (device_info(dev, &di) != 0) return hipErrorInvalidDevice;
  return hipMallocFromPoolAsync(p, bytes, di->pool, stream);
}
}  // namespace kda_host

extern "C" int kda_chunk_fwd(const void* q, const void* k, const void* v, const float* g,
                             const float* beta, const int32_t* cu_seqlens, int64_t T, int32_t H,
                             int32_t chunk, float gate_bound, void* out, hipStream_t stream) {
  t_last_error.clear();
  const kda_check::Result r =
      kda_check::chunk_fwd(q, k, v, g, beta, cu_seqlens, T, H, chunk, gate_bound, out);
  if (r.code != KDA_OK) return fail(r.code, r.msg);
  if (T == 0) return KDA_OK;
  const Call c{q, k, v, g, beta, cu_seqlens, T, H, gate_bound, out, -1, nullptr, nullptr, stream};
  return launch(c);
}

extern "C" int kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* g,
                                     const float* beta, const int32_t* cu_seqlens, int64_t T,
                                     int32_t H, int32_t chunk, float gate_bound, void* out,
                                     hipStream_t stream) {
  t_last_error.clear();
  const kda_check::Result r =
      kda_check::chunk_fwd(q, k, v, g, beta, cu_seqlens, T, H, chunk, gate_bound, out);
  if (r.code != KDA_OK) return fail(r.code, r.msg);
  if (T == 0) return KDA_OK;
  Call c{q, k, v, g, beta, cu_seqlens, T, H, gate_bound, out, -1, nullptr, nullptr, stream};
  c.no_alloc = true;
  return launch(c);
}

extern "C" int kda_chunk_fwd_state(const void* q, const void* k, const void* v, const float* g,
                                   const float* beta, const int32_t* cu_seqlens, int32_t n_docs,
                                   int64_t T, int32_t H, int32_t chunk, float gate_bound,
                                   const float* initial_state, float* final_state, void* out,
                                   hipStream_t stream) {
  t_last_error.clear();
  const kda_check::Result r =
      kda_check::chunk_fwd_state(q, k, v, g, beta, cu_seqlens, n_docs, T, H, chunk, gate_bound,
                                 initial_state, final_state, out);
  if (r.code != KDA_OK) return fail(r.code, r.msg);
  if (kda_check::fwd_is_noop(T, final_state)) return KDA_OK;
  const Call c{q, k, v, g, beta, cu_seqlens, T, H, gate_bound, out, n_docs, initial_state,
               final_state, stream};
  return launch(c);
}

extern "C" const char* kda_last_error(void) { return t_last_error.c_str(); }

extern "C" int kda_debug_set_split_policy(int policy) {
  if (policy < SPLIT_NEVER || policy > SPLIT_ALWAYS) return KDA_ERR_UNSUPPORTED;
  return g_split_policy.exchange(policy);
}

extern "C" int kda_device_status(hipStream_t stream) {
  if (hipStreamSynchronize(stream) != hipSuccess) return KDA_ERR_HIP;
  int st = 0;
  if (hipMemcpyFromSymbol(&st, HIP_SYMBOL(g_kda_status), sizeof(int), 0, hipMemcpyDeviceToHost) != hipSuccess)
    return KDA_ERR_HIP;
  const int zero = 0;
  if (hipMemcpyToSymbol(HIP_SYMBOL(g_kda_status), &zero, sizeof(int), 0, hipMemcpyHostToDevice) != hipSuccess)
    return KDA_ERR_HIP;
  return st;
}
