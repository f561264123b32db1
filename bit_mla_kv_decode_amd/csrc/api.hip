// C ABI of the gfx950 low-bit MLA cache library: argument validation, split
// selection, workspace layout and kernel launches.  See include/mla_lowbit.h
// for the contract of every entry point.
#include "mla_lowbit.h"

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "kernels.h"

// Device scratch of mla_decode_lowbit_noalloc: the decode's partial results
// (the workspace of mla_decode_lowbit) for callers that cannot allocate.
// Every device the library runs on holds its own copy until the process ends.
// Host code never passes `scratch` itself to a kernel (on the host it names a
// stand-in, not device memory): it uses the per-device address that
// hipGetSymbolAddress returns (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

mla_status_t fail(mla_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

// Compute units the decode plans for: the current device's count (256 on an
// MI355X), queried once per device, at most kMaxComputeUnits so that a
// sequence never has more balanced pieces than the combine kernel merges
// (two workgroups per unit: 512).  Without a device (host-only use of the
// size queries) the MI355X count is assumed.
constexpr int kMaxComputeUnits = 256;
constexpr int kMaxDevices = 64;
constexpr int kMaxSplits = 64;
constexpr int kMaxPagesPerSplit = 128;
// 2^24 pages = 2^30 tokens per sequence keeps every in-kernel token and
// per-64-sequence page count inside int32
constexpr int kMaxPagesPerSeq = 1 << 24;

int format_id(const mla_format_t* f) {
  if (!f) return -1;
  if (f->d_c != mla::kDc || f->d_r != mla::kDr || f->page_size != mla::kPage) return -1;
  if (f->c_bits == 4 && f->c_group == 64 && f->r_bits == 4 && f->r_group == 64) return mla::kC4R4;
  if (f->c_bits == 2 && f->c_group == 32 && f->r_bits == 4 && f->r_group == 64) return mla::kC2R4;
  if (f->c_bits == 16 && f->r_bits == 16) return mla::kBF16;
  return -1;
}

size_t page_bytes_of(int id) {
  switch (id) {
    case mla::kC4R4: return mla::PageLayout<mla::kC4R4>::kBytes;
    case mla::kC2R4: return mla::PageLayout<mla::kC2R4>::kBytes;
    case mla::kBF16: return mla::PageLayout<mla::kBF16>::kBytes;
    default: return 0;
  }
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int compute_units() {
  static std::atomic<int> known[kMaxDevices];  // 0: not queried yet
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return kMaxComputeUnits;
  int n = known[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1)
      v = kMaxComputeUnits;
    n = v < kMaxComputeUnits ? v : kMaxComputeUnits;
    known[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Workgroups that run at once: one per compute unit, two where the decode
// kernel splits channels over four wavefronts (17..32 rows per sequence,
// quantized formats).
int resident_groups(int fmt, int rows) { return compute_units() * mla::workgroups_per_cu(fmt, rows); }

// Partial-row slots: batch * splits per-sequence splits, or, for the balanced
// partition (splits == 0), one per (workgroup, sequence) piece: at most
// resident_groups + batch - 1.
size_t slot_count(int fmt, int batch, int rows, int splits) {
  return splits > 0 ? (size_t)batch * splits : (size_t)resident_groups(fmt, rows) + batch;
}

size_t partial_o_bytes(int fmt, int batch, int rows, int splits) {
  return align_up(slot_count(fmt, batch, rows, splits) * rows * mla::kDc * sizeof(float), 256);
}

size_t partial_lse_bytes(int fmt, int batch, int rows, int splits) {
  return align_up(slot_count(fmt, batch, rows, splits) * rows * sizeof(float), 256);
}

size_t workspace_bytes(int fmt, int batch, int rows, int splits) {
  size_t n = partial_o_bytes(fmt, batch, rows, splits) + partial_lse_bytes(fmt, batch, rows, splits);
  if (splits == 0) n += align_up((size_t)batch * 2 * sizeof(int), 256);  // per-sequence (first slot, count)
  return n;
}

int auto_splits(int fmt, int rows, int batch, int max_seq_len) {
  const int pages = (max_seq_len + mla::kPage - 1) / mla::kPage;
  if (batch <= 0 || pages <= 1) return 1;
  const int units = resident_groups(fmt, rows);
  int s = (units + batch - 1) / batch;                               // fill the compute units
  const int s_len = (pages + kMaxPagesPerSplit - 1) / kMaxPagesPerSplit;  // bound the longest split
  if (s_len > s) s = s_len;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s > pages) s = pages;
  return s < 1 ? 1 : s;
}

struct DecodeShape {
  int fmt;
  int splits;
  int pages_per_split;
  int s_q = 1;  // query tokens per sequence
};

// Query tokens per sequence accepted by the multi-token entry points.
constexpr int kMaxQueries = 16;

mla_status_t check_decode(const mla_format_t* fmt, const void* q, const void* cache, int64_t num_pages,
                          const int32_t* block_table, const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                          int32_t max_pages_per_seq, int32_t max_seq_len, float softmax_scale, int32_t num_splits,
                          DecodeShape* shape) {
  shape->fmt = format_id(fmt);
  if (shape->fmt < 0) return fail(MLA_ERR_UNSUPPORTED, "unsupported cache format");
  if (batch < 0) return fail(MLA_ERR_INVALID_ARG, "batch must be >= 0 (got %d)", batch);
  if (batch > 65535) return fail(MLA_ERR_UNSUPPORTED, "batch above 65535 is not supported (got %d)", batch);
  if (num_heads < 1 || num_heads > 128)
    return fail(MLA_ERR_UNSUPPORTED, "num_heads must be in 1..128 (got %d)", num_heads);
  if (max_pages_per_seq < 1) return fail(MLA_ERR_INVALID_ARG, "max_pages_per_seq must be >= 1");
  if (max_pages_per_seq > kMaxPagesPerSeq)
    return fail(MLA_ERR_UNSUPPORTED, "max_pages_per_seq above %d is not supported (got %d)", kMaxPagesPerSeq,
                max_pages_per_seq);
  if (num_pages < 1) return fail(MLA_ERR_INVALID_ARG, "num_pages must be >= 1");
  if (max_seq_len < 0) return fail(MLA_ERR_INVALID_ARG, "max_seq_len must be >= 0");
  if (!std::isfinite(softmax_scale)) return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be finite");
  if (num_splits < 0 || num_splits > kMaxSplits)
    return fail(MLA_ERR_INVALID_ARG, "num_splits must be in 0..%d (got %d)", kMaxSplits, num_splits);
  if (batch > 0) {
    if (!q || !cache || !block_table || !seq_lens) return fail(MLA_ERR_INVALID_ARG, "null tensor pointer");
    if (!aligned(q, 16) || !aligned(cache, 16))
      return fail(MLA_ERR_INVALID_ARG, "q and cache must be 16-byte aligned");
    if (!aligned(block_table, 4) || !aligned(seq_lens, 4))
      return fail(MLA_ERR_INVALID_ARG, "block_table and seq_lens must be 4-byte aligned");
  }
  int64_t cap = (int64_t)max_pages_per_seq * mla::kPage;
  int64_t hint = max_seq_len < cap ? max_seq_len : cap;
  shape->splits = num_splits;  // 0: balanced partition over the whole batch
  const int pages = (int)((hint + mla::kPage - 1) / mla::kPage);
  int pps = num_splits > 0 ? (pages + num_splits - 1) / num_splits : 1;
  shape->pages_per_split = pps < 1 ? 1 : pps;
  return MLA_OK;
}

mla::DecodeArgs make_args(const void* q, const void* cache, int64_t num_pages, const int32_t* block_table,
                          const int32_t* seq_lens, int32_t batch, int32_t num_heads, int32_t max_pages_per_seq,
                          float softmax_scale, const DecodeShape& sh, void* workspace) {
  mla::DecodeArgs a{};
  a.q = (const __bf16*)q;
  a.cache = (const uint8_t*)cache;
  a.num_pages = num_pages;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.heads = sh.s_q * num_heads;  // rows per sequence
  a.s_q = sh.s_q;
  a.qheads = num_heads;
  a.chunk_heads = num_heads < 128 / sh.s_q ? num_heads : 128 / sh.s_q;
  a.max_pages = max_pages_per_seq;
  a.num_splits = sh.splits;
  a.pages_per_split = sh.pages_per_split;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  if (workspace) {
    const int rows = sh.s_q * num_heads;
    a.o_part = (float*)workspace;
    a.lse_part = (float*)((char*)workspace + partial_o_bytes(sh.fmt, batch, rows, sh.splits));
    a.meta = (int*)((char*)workspace + partial_o_bytes(sh.fmt, batch, rows, sh.splits) +
                    partial_lse_bytes(sh.fmt, batch, rows, sh.splits));
  }
  return a;
}

// New-token rows for the fused append, or none.
struct Append {
  const void* latent = nullptr;
  const void* rope = nullptr;
  void* cache = nullptr;
};

void set_append(mla::DecodeArgs& a, const Append& ap) {
  a.new_latent = (const __bf16*)ap.latent;
  a.new_rope = (const __bf16*)ap.rope;
  a.append_cache = (uint8_t*)ap.cache;
}

mla_status_t decode_partial(const mla_format_t* fmt, const void* q_bf16, int32_t s_q, const void* cache,
                            int64_t num_pages, const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                            int32_t num_heads, int32_t max_pages_per_seq, int32_t max_seq_len, float softmax_scale,
                            int32_t num_splits, void* workspace, size_t ws_bytes, const Append& ap, void* stream) {
  DecodeShape sh;
  mla_status_t st = check_decode(fmt, q_bf16, cache, num_pages, block_table, seq_lens, batch, num_heads,
                                 max_pages_per_seq, max_seq_len, softmax_scale, num_splits, &sh);
  if (st != MLA_OK) return st;
  if (s_q < 1 || s_q > kMaxQueries)
    return fail(MLA_ERR_INVALID_ARG, "num_queries must be in 1..%d (got %d)", kMaxQueries, s_q);
  sh.s_q = s_q;
  if (batch == 0) return MLA_OK;
  const int rows = s_q * num_heads;
  if (!workspace || !aligned(workspace, 256))
    return fail(MLA_ERR_INVALID_ARG, "workspace must be a 256-byte aligned device pointer");
  if (ws_bytes < workspace_bytes(sh.fmt, batch, rows, sh.splits))
    return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes,
                workspace_bytes(sh.fmt, batch, rows, sh.splits));
  mla::DecodeArgs a = make_args(q_bf16, cache, num_pages, block_table, seq_lens, batch, num_heads,
                                max_pages_per_seq, softmax_scale, sh, workspace);
  set_append(a, ap);
  hipError_t e = sh.splits > 0 ? mla::launch_decode(sh.fmt, false, a, batch, (hipStream_t)stream)
                               : mla::launch_decode_flat(sh.fmt, a, resident_groups(sh.fmt, rows),
                                                         (hipStream_t)stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
  return MLA_OK;
}

// Device address of `scratch` on the current device, looked up on the first
// call on that device (with that device current) and kept per device.
mla_status_t noalloc_scratch(void** ptr) {
  static std::atomic<void*> known[kMaxDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MLA_ERR_UNSUPPORTED, "device %d: the no-allocation entry point serves devices 0..%d", dev,
                kMaxDevices - 1);
  void* p = known[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MLA_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    known[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return MLA_OK;
}

mla_status_t decode_combine(const mla_format_t* fmt, int32_t batch, int32_t num_heads, int32_t num_splits,
                            const void* workspace, size_t ws_bytes, void* out_bf16, float* lse_out, void* stream) {
  if (format_id(fmt) < 0) return fail(MLA_ERR_UNSUPPORTED, "unsupported cache format");
  if (batch < 0 || batch > 65535) return fail(MLA_ERR_INVALID_ARG, "batch must be in 0..65535");
  if (num_heads < 1 || num_heads > 128 * kMaxQueries)
    return fail(MLA_ERR_UNSUPPORTED, "rows per sequence (num_heads, times num_queries) must be in 1..%d",
                128 * kMaxQueries);
  if (num_splits < 0 || num_splits > kMaxSplits) return fail(MLA_ERR_INVALID_ARG, "num_splits must be in 0..64");
  if (batch == 0) return MLA_OK;
  if (!workspace || !out_bf16) return fail(MLA_ERR_INVALID_ARG, "null tensor pointer");
  if (!aligned(workspace, 256) || !aligned(out_bf16, 16) || (lse_out && !aligned(lse_out, 4)))
    return fail(MLA_ERR_INVALID_ARG, "misaligned workspace or output");
  const int id = format_id(fmt);
  if (ws_bytes < workspace_bytes(id, batch, num_heads, num_splits))
    return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes,
                workspace_bytes(id, batch, num_heads, num_splits));
  const float* o_part = (const float*)workspace;
  const float* lse_part =
      (const float*)((const char*)workspace + partial_o_bytes(id, batch, num_heads, num_splits));
  const int* meta = (const int*)((const char*)lse_part + partial_lse_bytes(id, batch, num_heads, num_splits));
  hipError_t e = num_splits > 0
                     ? mla::launch_combine(o_part, lse_part, batch, num_heads, num_splits, (__bf16*)out_bf16, lse_out,
                                           (hipStream_t)stream)
                     : mla::launch_combine_flat(o_part, lse_part, meta, batch, num_heads, (__bf16*)out_bf16, lse_out,
                                                (hipStream_t)stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "combine launch failed: %s", hipGetErrorString(e));
  return MLA_OK;
}

mla_status_t decode_full(const mla_format_t* fmt, const void* q_bf16, int32_t s_q, const void* cache,
                         int64_t num_pages, const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                         int32_t num_heads, int32_t max_pages_per_seq, int32_t max_seq_len, float softmax_scale,
                         int32_t num_splits, void* workspace, size_t ws_bytes, void* out_bf16, float* lse_out,
                         const Append& ap, void* stream) {
  DecodeShape sh;
  mla_status_t st = check_decode(fmt, q_bf16, cache, num_pages, block_table, seq_lens, batch, num_heads,
                                 max_pages_per_seq, max_seq_len, softmax_scale, num_splits, &sh);
  if (st != MLA_OK) return st;
  if (s_q < 1 || s_q > kMaxQueries)
    return fail(MLA_ERR_INVALID_ARG, "num_queries must be in 1..%d (got %d)", kMaxQueries, s_q);
  sh.s_q = s_q;
  if (batch == 0) return MLA_OK;
  if (!out_bf16 || !aligned(out_bf16, 16)) return fail(MLA_ERR_INVALID_ARG, "out must be a 16-byte aligned pointer");
  if (lse_out && !aligned(lse_out, 4)) return fail(MLA_ERR_INVALID_ARG, "lse_out must be 4-byte aligned");
  if (sh.splits == 1) {
    mla::DecodeArgs a = make_args(q_bf16, cache, num_pages, block_table, seq_lens, batch, num_heads,
                                  max_pages_per_seq, softmax_scale, sh, nullptr);
    a.out = (__bf16*)out_bf16;
    a.lse_out = lse_out;
    set_append(a, ap);
    hipError_t e = mla::launch_decode(sh.fmt, true, a, batch, (hipStream_t)stream);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
    return MLA_OK;
  }
  st = decode_partial(fmt, q_bf16, s_q, cache, num_pages, block_table, seq_lens, batch, num_heads,
                      max_pages_per_seq, max_seq_len, softmax_scale, sh.splits, workspace, ws_bytes, ap, stream);
  if (st != MLA_OK) return st;
  return decode_combine(fmt, batch, s_q * num_heads, sh.splits, workspace, ws_bytes, out_bf16, lse_out, stream);
}

}  // namespace

extern "C" {

size_t mla_token_bytes(const mla_format_t* fmt) { return page_bytes_of(format_id(fmt)) / mla::kPage; }

size_t mla_page_bytes(const mla_format_t* fmt) { return page_bytes_of(format_id(fmt)); }

const char* mla_last_error(void) { return g_err; }

mla_status_t mla_quant_append(const mla_format_t* fmt, const void* latent_bf16, const void* rope_bf16,
                              const int32_t* slot_mapping, int32_t n_new, void* cache, int64_t num_pages,
                              void* stream) {
  const int id = format_id(fmt);
  if (id < 0) return fail(MLA_ERR_UNSUPPORTED, "unsupported cache format");
  if (n_new < 0) return fail(MLA_ERR_INVALID_ARG, "n_new must be >= 0 (got %d)", n_new);
  if (n_new == 0) return MLA_OK;
  if (!latent_bf16 || !rope_bf16 || !slot_mapping || !cache) return fail(MLA_ERR_INVALID_ARG, "null tensor pointer");
  if (num_pages < 1) return fail(MLA_ERR_INVALID_ARG, "num_pages must be >= 1");
  if (!aligned(latent_bf16, 16) || !aligned(rope_bf16, 16) || !aligned(cache, 16))
    return fail(MLA_ERR_INVALID_ARG, "latent, rope and cache must be 16-byte aligned");
  if (!aligned(slot_mapping, 4)) return fail(MLA_ERR_INVALID_ARG, "slot_mapping must be 4-byte aligned");
  hipError_t e = mla::launch_quant_append(id, latent_bf16, rope_bf16, slot_mapping, n_new, cache, num_pages,
                                          (hipStream_t)stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "quant_append launch failed: %s", hipGetErrorString(e));
  return MLA_OK;
}

int32_t mla_decode_num_splits(const mla_format_t* fmt, int32_t batch, int32_t num_heads, int32_t max_seq_len) {
  const int id = format_id(fmt);
  return auto_splits(id < 0 ? mla::kBF16 : id, num_heads, batch, max_seq_len);
}

size_t mla_decode_workspace_bytes(const mla_format_t* fmt, int32_t batch, int32_t num_heads, int32_t num_splits) {
  if (format_id(fmt) < 0 || batch < 0 || num_heads < 1 || num_splits < 0 || num_splits > kMaxSplits) return 0;
  return workspace_bytes(format_id(fmt), batch, num_heads, num_splits);
}

int64_t mla_decode_partial_slots(const mla_format_t* fmt, int32_t batch, int32_t num_heads, int32_t num_splits) {
  if (format_id(fmt) < 0 || batch < 0 || num_heads < 1 || num_splits < 0 || num_splits > kMaxSplits) return 0;
  return (int64_t)slot_count(format_id(fmt), batch, num_heads, num_splits);
}

mla_status_t mla_decode_partial(const mla_format_t* fmt, const void* q_bf16, const void* cache, int64_t num_pages,
                                const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                                int32_t num_heads, int32_t max_pages_per_seq, int32_t max_seq_len,
                                float softmax_scale, int32_t num_splits, void* workspace, size_t ws_bytes,
                                void* stream) {
  return decode_partial(fmt, q_bf16, 1, cache, num_pages, block_table, seq_lens, batch, num_heads, max_pages_per_seq,
                        max_seq_len, softmax_scale, num_splits, workspace, ws_bytes, Append{}, stream);
}

mla_status_t mla_decode_combine(const mla_format_t* fmt, int32_t batch, int32_t num_heads, int32_t num_splits,
                                const void* workspace, size_t ws_bytes, void* out_bf16, float* lse_out,
                                void* stream) {
  return decode_combine(fmt, batch, num_heads, num_splits, workspace, ws_bytes, out_bf16, lse_out, stream);
}

mla_status_t mla_decode_lowbit(const mla_format_t* fmt, const void* q_bf16, const void* cache, int64_t num_pages,
                               const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                               int32_t num_heads, int32_t max_pages_per_seq, int32_t max_seq_len,
                               float softmax_scale, int32_t num_splits, void* workspace, size_t ws_bytes,
                               void* out_bf16, float* lse_out, void* stream) {
  return decode_full(fmt, q_bf16, 1, cache, num_pages, block_table, seq_lens, batch, num_heads, max_pages_per_seq,
                     max_seq_len, softmax_scale, num_splits, workspace, ws_bytes, out_bf16, lse_out, Append{}, stream);
}

mla_status_t mla_decode_lowbit_noalloc(const mla_format_t* fmt, const void* q_bf16, const void* cache,
                                       int64_t num_pages, const int32_t* block_table, const int32_t* seq_lens,
                                       int32_t batch, int32_t num_heads, int32_t max_pages_per_seq,
                                       int32_t max_seq_len, float softmax_scale, int32_t num_splits, void* out_bf16,
                                       float* lse_out, void* stream) {
  DecodeShape sh;
  mla_status_t st = check_decode(fmt, q_bf16, cache, num_pages, block_table, seq_lens, batch, num_heads,
                                 max_pages_per_seq, max_seq_len, softmax_scale, num_splits, &sh);
  if (st != MLA_OK || batch == 0) return st;
  void* ws = nullptr;
  if (num_splits != 1) {  // one split writes the output directly: no scratch
    const size_t need = workspace_bytes(sh.fmt, batch, num_heads, num_splits);
    if (need > (size_t)MLA_NOALLOC_SCRATCH_BYTES)
      return fail(MLA_ERR_WORKSPACE,
                  "this shape needs %zu bytes of decode scratch; the no-allocation entry point holds %zu per device "
                  "(use fewer sequences per call, fixed splits, or mla_decode_lowbit with a workspace)",
                  need, (size_t)MLA_NOALLOC_SCRATCH_BYTES);
    st = noalloc_scratch(&ws);
    if (st != MLA_OK) return st;
  }
  return decode_full(fmt, q_bf16, 1, cache, num_pages, block_table, seq_lens, batch, num_heads, max_pages_per_seq,
                     max_seq_len, softmax_scale, num_splits, ws, ws ? (size_t)MLA_NOALLOC_SCRATCH_BYTES : 0,
                     out_bf16, lse_out, Append{}, stream);
}

mla_status_t mla_decode_append_partial(const mla_format_t* fmt, const void* latent_new_bf16,
                                       const void* rope_new_bf16, const void* q_bf16, void* cache, int64_t num_pages,
                                       const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                                       int32_t num_heads, int32_t max_pages_per_seq, int32_t max_seq_len,
                                       float softmax_scale, int32_t num_splits, void* workspace, size_t ws_bytes,
                                       void* stream) {
  if (batch > 0) {
    if (!latent_new_bf16 || !rope_new_bf16) return fail(MLA_ERR_INVALID_ARG, "null new-row pointer");
    if (!aligned(latent_new_bf16, 16) || !aligned(rope_new_bf16, 16))
      return fail(MLA_ERR_INVALID_ARG, "new latent and rope rows must be 16-byte aligned");
  }
  Append ap;
  ap.latent = latent_new_bf16;
  ap.rope = rope_new_bf16;
  ap.cache = cache;
  return decode_partial(fmt, q_bf16, 1, cache, num_pages, block_table, seq_lens, batch, num_heads, max_pages_per_seq,
                        max_seq_len, softmax_scale, num_splits, workspace, ws_bytes, ap, stream);
}

mla_status_t mla_decode_append_lowbit(const mla_format_t* fmt, const void* latent_new_bf16, const void* rope_new_bf16,
                                      const void* q_bf16, void* cache, int64_t num_pages, const int32_t* block_table,
                                      const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                                      int32_t max_pages_per_seq, int32_t max_seq_len, float softmax_scale,
                                      int32_t num_splits, void* workspace, size_t ws_bytes, void* out_bf16,
                                      float* lse_out, void* stream) {
  if (batch > 0) {
    if (!latent_new_bf16 || !rope_new_bf16) return fail(MLA_ERR_INVALID_ARG, "null new-row pointer");
    if (!aligned(latent_new_bf16, 16) || !aligned(rope_new_bf16, 16))
      return fail(MLA_ERR_INVALID_ARG, "new latent and rope rows must be 16-byte aligned");
  }
  Append ap;
  ap.latent = latent_new_bf16;
  ap.rope = rope_new_bf16;
  ap.cache = cache;
  return decode_full(fmt, q_bf16, 1, cache, num_pages, block_table, seq_lens, batch, num_heads, max_pages_per_seq,
                     max_seq_len, softmax_scale, num_splits, workspace, ws_bytes, out_bf16, lse_out, ap, stream);
}

mla_status_t mla_decode_multi_lowbit(const mla_format_t* fmt, const void* q_bf16, int32_t num_queries,
                                     const void* cache, int64_t num_pages, const int32_t* block_table,
                                     const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                                     int32_t max_pages_per_seq, int32_t max_seq_len, float softmax_scale,
                                     int32_t num_splits, void* workspace, size_t ws_bytes, void* out_bf16,
                                     float* lse_out, void* stream) {
  return decode_full(fmt, q_bf16, num_queries, cache, num_pages, block_table, seq_lens, batch, num_heads,
                     max_pages_per_seq, max_seq_len, softmax_scale, num_splits, workspace, ws_bytes, out_bf16, lse_out,
                     Append{}, stream);
}

mla_status_t mla_decode_multi_partial(const mla_format_t* fmt, const void* q_bf16, int32_t num_queries,
                                      const void* cache, int64_t num_pages, const int32_t* block_table,
                                      const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                                      int32_t max_pages_per_seq, int32_t max_seq_len, float softmax_scale,
                                      int32_t num_splits, void* workspace, size_t ws_bytes, void* stream) {
  return decode_partial(fmt, q_bf16, num_queries, cache, num_pages, block_table, seq_lens, batch, num_heads,
                        max_pages_per_seq, max_seq_len, softmax_scale, num_splits, workspace, ws_bytes, Append{},
                        stream);
}

mla_status_t mla_absorb_q(const void* q_nope_bf16, const void* q_pe_bf16, const void* w_uk_bf16, int32_t batch,
                          int32_t num_heads, void* q_out_bf16, void* stream) {
  if (batch < 0) return fail(MLA_ERR_INVALID_ARG, "batch must be >= 0 (got %d)", batch);
  if (num_heads < 1 || num_heads > 1024) return fail(MLA_ERR_UNSUPPORTED, "num_heads must be in 1..1024");
  if (batch == 0) return MLA_OK;
  if (!q_nope_bf16 || !q_pe_bf16 || !w_uk_bf16 || !q_out_bf16) return fail(MLA_ERR_INVALID_ARG, "null tensor pointer");
  if (!aligned(q_nope_bf16, 16) || !aligned(w_uk_bf16, 16) || !aligned(q_out_bf16, 16) || !aligned(q_pe_bf16, 2))
    return fail(MLA_ERR_INVALID_ARG, "q_nope, w_uk and q_out must be 16-byte aligned");
  hipError_t e = mla::launch_absorb_q(q_nope_bf16, q_pe_bf16, w_uk_bf16, batch, num_heads, q_out_bf16,
                                      (hipStream_t)stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "absorb launch failed: %s", hipGetErrorString(e));
  return MLA_OK;
}

mla_status_t mla_project_out(const void* latent_bf16, const void* w_uv_bf16, int32_t batch, int32_t num_heads,
                             void* out_bf16, void* stream) {
  if (batch < 0) return fail(MLA_ERR_INVALID_ARG, "batch must be >= 0 (got %d)", batch);
  if (num_heads < 1 || num_heads > 1024) return fail(MLA_ERR_UNSUPPORTED, "num_heads must be in 1..1024");
  if (batch == 0) return MLA_OK;
  if (!latent_bf16 || !w_uv_bf16 || !out_bf16) return fail(MLA_ERR_INVALID_ARG, "null tensor pointer");
  if (!aligned(latent_bf16, 16) || !aligned(w_uv_bf16, 16) || !aligned(out_bf16, 2))
    return fail(MLA_ERR_INVALID_ARG, "latent and w_uv must be 16-byte aligned");
  hipError_t e = mla::launch_project_out(latent_bf16, w_uv_bf16, batch, num_heads, out_bf16, (hipStream_t)stream);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "projection launch failed: %s", hipGetErrorString(e));
  return MLA_OK;
}

}  // extern "C"
