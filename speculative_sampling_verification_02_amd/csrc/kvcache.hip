// KV-cache crop after a verification step, for gfx950.
//
// [FI] "The loop: draft, verify in one pass, keep a prefix" (its KV-cache
// paragraph): the verification pass appends the drafts' entries to the
// target's cache, and after the accept test the entries past the accepted
// prefix are discarded -- one crop after the sampling function.  [LH] "Fix the
// benchmark conditions first": the cache follows the committed prefix, and
// with paged storage the rejected state is whole pages, returned to the pool.
//
// Sequence b had seq_len[b] committed entries before the verification pass,
// which wrote `appended` more.  The crop keeps keep_extra of those plus one
// per accepted draft: new_len = seq_len[b] + keep_extra + n_accepted[b].  A
// sequence whose verification reported -1 is left as it was.  n_accepted is
// read on the device, so the crop queues right after the verification on the
// same stream with no host synchronisation.
//
// Two launches:
//   clear    (optional) zero-fills the discarded entries [new_len, seq_len +
//            appended) of every cache with 16-byte stores: one workgroup per
//            sequence and group of 8 caches, its rows (or paged slots) taken
//            as one flat range of words;
//   lengths  the new lengths -- for paged storage one workgroup that also
//            releases every page past the new length: table entry to -1, page
//            id appended to the free list in sequence order, then block order,
//            through a workgroup scan of the per-sequence counts, so the list
//            is the same on every run.
// The clear reads the old lengths and block tables, so it runs first.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specverify.h"

namespace {

constexpr int kClearThreads = 256;
constexpr int kFinishThreads = 1024;
constexpr int kMaxCaches = SPEC_KV_MAX_CACHES;
constexpr int kCachesPerGroup = 8;                  // caches one clearing workgroup covers
constexpr int kMaxAppended = SPEC_KV_MAX_APPENDED;  // paged: discarded slots one workgroup looks up

struct CacheList {
  char* p[kMaxCaches];
};

struct Crop {
  int B;
  int appended, keep_extra;
  int32_t* seq_len;
  const int32_t* n_acc;
  // contiguous: [B][H][S_max][entry_bytes]
  int H, S_max;
  long long entry_bytes;
  // paged: [num_pages][page_size][token_bytes], block_table [B][max_blocks]
  int num_pages, page_size, max_blocks;
  long long token_bytes;
  int32_t* table;
  int32_t* free_pages;
  int32_t* free_count;
  int free_capacity;
};

// [lo, hi) of the discarded positions of sequence b (lo >= hi: nothing), or
// false for a sequence left as it was.
__device__ inline bool discarded(const Crop& c, int b, long long* lo, long long* hi) {
  const int n = c.n_acc[b];
  if (n < 0) return false;
  const long long base = c.seq_len[b];
  *lo = base + c.keep_extra + n;
  *hi = base + c.appended;
  return true;
}

// Zero `nrows` rows of `row_words` 16-byte words each; row r starts at word
// row_start(r) of cache row_cache(r).  Rows shorter than the workgroup are
// packed several to a pass, so a thread's row and word offsets are fixed for
// the whole loop (no division per store).
template <class RowAddr>
__device__ inline void zero_rows(int nrows, int row_words, RowAddr row_addr) {
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  const int t = threadIdx.x;
  if (row_words >= kClearThreads) {
    for (int r = 0; r < nrows; ++r) {
      uint4* row = row_addr(r);
      for (int w = t; w < row_words; w += kClearThreads) row[w] = z;
    }
    return;
  }
  const int per_pass = kClearThreads / row_words;  // rows per pass
  const int my_row = t / row_words, my_word = t - my_row * row_words;
  if (my_row >= per_pass) return;
  for (int r = my_row; r < nrows; r += per_pass) row_addr(r)[my_word] = z;
}

// grid (B, ceil(n_caches / kCachesPerGroup)): sequence b's discarded rows
// (one per cache and head) in a group of caches.
__global__ __launch_bounds__(kClearThreads) void clear_contiguous(Crop c, CacheList caches, int n_caches) {
  const int b = blockIdx.x;
  long long lo, hi;
  if (!discarded(c, b, &lo, &hi)) return;
  lo = lo < 0 ? 0 : (lo > c.S_max ? c.S_max : lo);
  hi = hi < 0 ? 0 : (hi > c.S_max ? c.S_max : hi);
  if (lo >= hi) return;
  const int c0 = blockIdx.y * kCachesPerGroup;
  const int nc = min(kCachesPerGroup, n_caches - c0);
  const int row_words = (int)((hi - lo) * (c.entry_bytes / 16));  // at most S_max * entry_bytes / 16
  const long long head_stride = (long long)c.S_max * (c.entry_bytes / 16);
  const long long start = ((long long)b * c.H * c.S_max + lo) * (c.entry_bytes / 16);
  const int H = c.H;
  zero_rows(nc * H, row_words, [&](int r) {
    const int ci = r / H, h = r - ci * H;
    return reinterpret_cast<uint4*>(caches.p[c0 + ci]) + start + h * head_stride;
  });
}

// grid (B, ceil(n_caches / kCachesPerGroup)): sequence b's discarded slots in
// a group of caches.  The slots' page addresses are looked up once into LDS.
__global__ __launch_bounds__(kClearThreads) void clear_paged(Crop c, CacheList caches, int n_caches) {
  __shared__ long long slot_word[kMaxAppended];  // first word of each discarded slot, -1: no page
  __shared__ int nslots;
  const int b = blockIdx.x;
  long long lo, hi;
  if (!discarded(c, b, &lo, &hi)) return;
  lo = lo < 0 ? 0 : lo;
  const int npos = (int)(hi > lo ? hi - lo : 0);  // at most `appended`
  if (npos <= 0) return;
  const long long token_words = c.token_bytes / 16;
  if (threadIdx.x == 0) {
    // the slots that lie in a page of these caches, in position order
    int n = 0;
    for (int k = 0; k < npos; ++k) {
      const long long s = lo + k, j = s / c.page_size;
      const int page = j < c.max_blocks ? c.table[(long long)b * c.max_blocks + j] : -1;
      // an entry outside [0, num_pages) is not a page of these caches
      if (page >= 0 && page < c.num_pages) slot_word[n++] = ((long long)page * c.page_size + s % c.page_size) * token_words;
    }
    nslots = n;
  }
  __syncthreads();
  const int c0 = blockIdx.y * kCachesPerGroup;
  const int nc = min(kCachesPerGroup, n_caches - c0);
  const int ns = nslots;
  zero_rows(nc * ns, (int)token_words, [&](int r) {
    const int ci = r / ns, k = r - ci * ns;
    return reinterpret_cast<uint4*>(caches.p[c0 + ci]) + slot_word[k];
  });
}

// Contiguous caches: the new lengths (a sequence with -1 is left as it was).
__global__ __launch_bounds__(kClearThreads) void update_lengths(Crop c) {
  const int b = blockIdx.x * kClearThreads + threadIdx.x;
  long long lo, hi;
  if (b < c.B && discarded(c, b, &lo, &hi)) c.seq_len[b] = (int32_t)lo;
}

// Exclusive scan of one int per thread over the workgroup (Hillis-Steele in
// LDS); *total gets the sum.
__device__ inline int block_exclusive_scan(int v, int* lds, int* total) {
  const int t = threadIdx.x;
  lds[t] = v;
  __syncthreads();
  for (int off = 1; off < kFinishThreads; off <<= 1) {
    const int add = t >= off ? lds[t - off] : 0;
    __syncthreads();
    lds[t] += add;
    __syncthreads();
  }
  const int incl = lds[t];
  *total = lds[kFinishThreads - 1];
  __syncthreads();
  return incl - v;
}

// Paged caches, one workgroup of kFinishThreads: the new lengths and the
// release of the pages past them.
__global__ __launch_bounds__(kFinishThreads) void release_pages(Crop c) {
  __shared__ int lds[kFinishThreads];
  int base = *c.free_count;  // read by every thread before thread 0 writes it (below)
  for (int b0 = 0; b0 < c.B; b0 += kFinishThreads) {
    const int b = b0 + (int)threadIdx.x;
    long long lo = 0, hi = 0;
    const bool live = b < c.B && discarded(c, b, &lo, &hi);
    long long first = 0;
    int count = 0;
    if (live) {
      const long long keep = lo <= 0 ? 0 : (lo + c.page_size - 1) / c.page_size;
      first = keep;
      for (long long j = keep; j < c.max_blocks; ++j) count += c.table[(long long)b * c.max_blocks + j] >= 0;
    }
    int total = 0;
    const int excl = block_exclusive_scan(count, lds, &total);
    if (live && count) {
      int k = base + excl;
      for (long long j = first; j < c.max_blocks; ++j) {
        int32_t* e = c.table + (long long)b * c.max_blocks + j;
        if (*e < 0) continue;
        if (k < c.free_capacity) c.free_pages[k] = *e;
        ++k;
        *e = -1;
      }
    }
    if (live) c.seq_len[b] = (int32_t)lo;
    base += total;
  }
  __syncthreads();
  if (threadIdx.x == 0) *c.free_count = base;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int map_hip(hipError_t e) { return e == hipSuccess ? SPEC_OK : SPEC_EHIP; }

bool fill_caches(void* const* caches, int n_caches, int clear, CacheList* out) {
  if (!clear) return true;
  if (!caches || n_caches < 1 || n_caches > kMaxCaches) return false;
  for (int i = 0; i < n_caches; ++i) {
    if (!caches[i] || !aligned16(caches[i])) return false;
    out->p[i] = static_cast<char*>(caches[i]);
  }
  return true;
}

}  // namespace

extern "C" {

int spec_kv_crop(void* const* caches, int n_caches, int B, int H, int S_max, int entry_bytes, int32_t* seq_len,
                 const int32_t* n_accepted, int appended, int keep_extra, int clear, void* stream) {
  if (B < 0 || H < 1 || S_max < 1 || entry_bytes < 16 || entry_bytes % 16 != 0) return SPEC_EINVAL;
  if ((long long)S_max * (entry_bytes / 16) > INT32_MAX) return SPEC_EINVAL;  // one row's words fit an int
  if (appended < 0 || keep_extra < 0 || keep_extra > appended) return SPEC_EINVAL;
  if (B == 0) return SPEC_OK;
  if (!seq_len || !n_accepted) return SPEC_EINVAL;
  CacheList list{};
  if (!fill_caches(caches, n_caches, clear, &list)) return SPEC_EINVAL;
  Crop c{};
  c.B = B;
  c.appended = appended;
  c.keep_extra = keep_extra;
  c.seq_len = seq_len;
  c.n_acc = n_accepted;
  c.H = H;
  c.S_max = S_max;
  c.entry_bytes = entry_bytes;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned groups = (unsigned)((n_caches + kCachesPerGroup - 1) / kCachesPerGroup);
  if (clear && appended > 0)
    clear_contiguous<<<dim3((unsigned)B, groups), dim3(kClearThreads), 0, s>>>(c, list, n_caches);
  update_lengths<<<dim3((unsigned)((B + kClearThreads - 1) / kClearThreads)), dim3(kClearThreads), 0, s>>>(c);
  return map_hip(hipGetLastError());
}

int spec_kv_crop_paged(void* const* caches, int n_caches, int num_pages, int page_size, int token_bytes,
                       int32_t* block_table, int B, int max_blocks, int32_t* seq_len, const int32_t* n_accepted,
                       int appended, int keep_extra, int clear, int32_t* free_pages, int32_t* free_count,
                       int free_capacity, void* stream) {
  if (B < 0 || num_pages < 1 || page_size < 1 || max_blocks < 1) return SPEC_EINVAL;
  if (token_bytes < 16 || token_bytes % 16 != 0) return SPEC_EINVAL;
  if (appended < 0 || appended > kMaxAppended || keep_extra < 0 || keep_extra > appended) return SPEC_EINVAL;
  if (free_capacity < num_pages) return SPEC_EINVAL;
  if (B == 0) return SPEC_OK;
  if (!block_table || !seq_len || !n_accepted || !free_pages || !free_count) return SPEC_EINVAL;
  CacheList list{};
  if (!fill_caches(caches, n_caches, clear, &list)) return SPEC_EINVAL;
  Crop c{};
  c.B = B;
  c.appended = appended;
  c.keep_extra = keep_extra;
  c.seq_len = seq_len;
  c.n_acc = n_accepted;
  c.num_pages = num_pages;
  c.page_size = page_size;
  c.max_blocks = max_blocks;
  c.token_bytes = token_bytes;
  c.table = block_table;
  c.free_pages = free_pages;
  c.free_count = free_count;
  c.free_capacity = free_capacity;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned groups = (unsigned)((n_caches + kCachesPerGroup - 1) / kCachesPerGroup);
  if (clear && appended > 0)
    clear_paged<<<dim3((unsigned)B, groups), dim3(kClearThreads), 0, s>>>(c, list, n_caches);
  release_pages<<<dim3(1), dim3(kFinishThreads), 0, s>>>(c);
  return map_hip(hipGetLastError());
}

}  // extern "C"
