// HPTQ's stored form: the integer levels of a layer as one Huffman-coded bit
// stream (The Geometry of LLM Quantization, section 3: inliers and outliers
// share one unbounded integer grid, and the integers are Huffman-coded).
//
// Encoding: a level histogram on the device; on the host the Huffman code
// lengths (two lightest subtrees merged first; ties: the node made earlier,
// leaves in increasing level order) and the canonical code (symbols ordered
// by length, then level; each code the previous one plus one, shifted by the
// growth in length); per row the sum of its code lengths (one wave per row),
// one workgroup's scan over the rows gives every row's first bit, then one
// wave per row writes its codes in column order: a wave prefix sum of the 64
// lengths gives each code's position, and the code bits go into the 32-bit
// words they span with atomic ORs (most significant code bit first; bit b of
// the stream is bit 31 - b % 32 of word b / 32). Decoding: one thread per row
// reads its bits from the row's first bit and matches them against the
// canonical code one bit at a time.
#include <algorithm>
#include <queue>
#include <vector>

#include "common.h"

namespace gptq {

constexpr int HF_SYMS = 65536;  // int16 levels, at level + 32768
constexpr int HF_MAXLEN = 63;   // longest code handled

struct HFLayout {
  size_t hist, len, code, first, count, index, sorted, total;
  HFLayout() {
    size_t p = 0;
    auto take = [&](size_t bytes) {
      const size_t at = p;
      p = (size_t)round_up((int64_t)(p + bytes), 256);
      return at;
    };
    hist = take(4 * (size_t)HF_SYMS);
    len = take((size_t)HF_SYMS);
    code = take(8 * (size_t)HF_SYMS);
    first = take(8 * (HF_MAXLEN + 2));
    count = take(4 * (HF_MAXLEN + 2));
    index = take(4 * (HF_MAXLEN + 2));
    sorted = take(2 * (size_t)HF_SYMS);
    total = p;
  }
};

__global__ void hf_zero_kernel(unsigned* __restrict__ p, int64_t n) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x)
    p[e] = 0u;
}

// level histogram: levels in [-1024, 1023] counted in LDS first (the common
// ones), the others straight into the global bins
constexpr int HF_LDS = 2048;
__global__ __launch_bounds__(256) void hf_hist_kernel(const int16_t* __restrict__ lv, int64_t n,
                                                      unsigned* __restrict__ hist) {
  __shared__ unsigned hl[HF_LDS];
  for (int i = threadIdx.x; i < HF_LDS; i += blockDim.x) hl[i] = 0u;
  __syncthreads();
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int k = lv[e];
    if (k >= -HF_LDS / 2 && k < HF_LDS / 2) atomicAdd(&hl[k + HF_LDS / 2], 1u);
    else atomicAdd(&hist[k + 32768], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < HF_LDS; i += blockDim.x)
    if (hl[i]) atomicAdd(&hist[i - HF_LDS / 2 + 32768], hl[i]);
}

// bits of row r: the sum of its code lengths (one wave per row)
__global__ __launch_bounds__(256) void hf_rowbits_kernel(const int16_t* __restrict__ lv,
                                                         int64_t rows, int64_t cols,
                                                         const uint8_t* __restrict__ len,
                                                         int64_t* __restrict__ row_bit) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  int64_t b = 0;
  for (int64_t c = lane; c < cols; c += 64) b += len[(int)lv[r * cols + c] + 32768];
  for (int off = 32; off > 0; off >>= 1) b += __shfl_xor(b, off, 64);
  if (lane == 0) row_bit[r + 1] = b;
}

// inclusive scan of row_bit[1..rows] in place, row_bit[0] = 0 (one workgroup)
__global__ __launch_bounds__(1024) void hf_scan_kernel(int64_t* __restrict__ row_bit,
                                                       int64_t rows) {
  __shared__ int64_t part[16];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  if (t == 0) row_bit[0] = 0;
  int64_t carry = 0;
  for (int64_t base = 0; base < rows; base += 1024) {
    const int64_t r = base + t;
    int64_t v = r < rows ? row_bit[r + 1] : 0;
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t y = __shfl_up(v, off, 64);
      if (lane >= off) v += y;
    }
    if (lane == 63) part[w] = v;
    __syncthreads();
    int64_t before = carry;
    for (int k = 0; k < w; ++k) before += part[k];
    int64_t total = carry;
    for (int k = 0; k < 16; ++k) total += part[k];
    if (r < rows) row_bit[r + 1] = before + v;
    __syncthreads();
    carry = total;
  }
}

// OR the `ln` low bits of `code` into the stream at bit position `pos`
__device__ inline void hf_put(uint32_t* __restrict__ words, int64_t pos, uint64_t code, int ln) {
  while (ln > 0) {
    const int64_t wi = pos >> 5;
    const int off = (int)(pos & 31);   // bits of this word before the code
    const int take = ln < 32 - off ? ln : 32 - off;
    const uint32_t chunk = (uint32_t)((code >> (ln - take)) & ((1ull << take) - 1));
    atomicOr(&words[wi], chunk << (32 - off - take));
    pos += take;
    ln -= take;
  }
}

__global__ __launch_bounds__(256) void hf_encode_kernel(const int16_t* __restrict__ lv,
                                                        int64_t rows, int64_t cols,
                                                        const uint8_t* __restrict__ len,
                                                        const uint64_t* __restrict__ code,
                                                        const int64_t* __restrict__ row_bit,
                                                        uint32_t* __restrict__ words) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  int64_t pos = row_bit[r];
  for (int64_t c0 = 0; c0 < cols; c0 += 64) {
    const int64_t c = c0 + lane;
    int ln = 0;
    uint64_t cd = 0;
    if (c < cols) {
      const int s = (int)lv[r * cols + c] + 32768;
      ln = len[s];
      cd = code[s];
    }
    // exclusive prefix sum of the lengths over the wave
    int64_t incl = ln;
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (ln > 0) hf_put(words, pos + incl - ln, cd, ln);
    pos += __shfl(incl, 63, 64);
  }
}

// one thread per row: canonical decoding, bit by bit
__global__ __launch_bounds__(256) void hf_decode_kernel(
    const uint32_t* __restrict__ words, int64_t nwords, const int64_t* __restrict__ row_bit,
    int64_t rows, int64_t cols, const uint64_t* __restrict__ first, const int* __restrict__ count,
    const int* __restrict__ index, const int16_t* __restrict__ sorted, int16_t* __restrict__ lv,
    unsigned* __restrict__ bad) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  int64_t b = row_bit[r];
  for (int64_t c = 0; c < cols; ++c) {
    uint64_t cd = 0;
    int ln = 0;
    int16_t sym = 0;
    bool found = false;
    while (!found && ln < HF_MAXLEN && (b >> 5) < nwords) {
      const uint32_t bit = (words[b >> 5] >> (31 - (int)(b & 31))) & 1u;
      cd = (cd << 1) | bit;
      ++ln;
      ++b;
      if (count[ln] > 0 && cd >= first[ln] && cd - first[ln] < (uint64_t)count[ln]) {
        sym = sorted[index[ln] + (int)(cd - first[ln])];
        found = true;
      }
    }
    if (!found) {
      atomicOr(bad, 1u);
      return;
    }
    lv[r * cols + c] = sym;
  }
}

// Huffman code lengths of the histogram (0 for absent levels): repeatedly
// merge the two lightest subtrees, ties to the one made earlier (leaves in
// increasing level order come first); a single level gets length 1.
static bool hf_lengths(const std::vector<unsigned>& h, std::vector<uint8_t>& len) {
  len.assign(HF_SYMS, 0);
  struct Node {
    uint64_t w;
    int id;
  };
  auto later = [](const Node& a, const Node& b) { return a.w != b.w ? a.w > b.w : a.id > b.id; };
  std::priority_queue<Node, std::vector<Node>, decltype(later)> pq(later);
  std::vector<int> parent;
  std::vector<int> leaf_sym;
  for (int s = 0; s < HF_SYMS; ++s)
    if (h[s]) {
      pq.push({h[s], (int)parent.size()});
      parent.push_back(-1);
      leaf_sym.push_back(s);
    }
  const int nleaf = (int)leaf_sym.size();
  if (nleaf == 0) return true;
  if (nleaf == 1) {
    len[leaf_sym[0]] = 1;
    return true;
  }
  while (pq.size() > 1) {
    const Node a = pq.top();
    pq.pop();
    const Node b = pq.top();
    pq.pop();
    const int id = (int)parent.size();
    parent.push_back(-1);
    parent[a.id] = id;
    parent[b.id] = id;
    pq.push({a.w + b.w, id});
  }
  // depth of every node, from the root (the last node) down
  std::vector<int> depth(parent.size(), 0);
  for (int v = (int)parent.size() - 2; v >= 0; --v) depth[v] = depth[parent[v]] + 1;
  for (int i = 0; i < nleaf; ++i) {
    if (depth[i] > HF_MAXLEN) return false;
    len[leaf_sym[i]] = (uint8_t)depth[i];
  }
  return true;
}

// canonical code and decoding tables from the lengths
static void hf_canonical(const std::vector<uint8_t>& len, std::vector<uint64_t>& code,
                         std::vector<uint64_t>& first, std::vector<int>& count,
                         std::vector<int>& index, std::vector<int16_t>& sorted) {
  code.assign(HF_SYMS, 0);
  first.assign(HF_MAXLEN + 2, 0);
  count.assign(HF_MAXLEN + 2, 0);
  index.assign(HF_MAXLEN + 2, 0);
  sorted.clear();
  std::vector<int> order;
  for (int s = 0; s < HF_SYMS; ++s)
    if (len[s]) order.push_back(s);
  // by length, then level (symbol s is level s - 32768, so s orders levels;
  // the stable sort keeps that order within a length)
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return len[a] < len[b]; });
  uint64_t c = 0;
  int prev = order.empty() ? 0 : len[order[0]];
  for (size_t i = 0; i < order.size(); ++i) {
    const int s = order[i], l = len[s];
    if (i > 0) c = (c + 1) << (l - prev);
    code[s] = c;
    if (count[l] == 0) {
      first[l] = c;
      index[l] = (int)i;
    }
    ++count[l];
    sorted.push_back((int16_t)(s - 32768));
    prev = l;
  }
}

}  // namespace gptq

using namespace gptq;

extern "C" size_t gptq_hptq_code_workspace_bytes(void) { return HFLayout().total; }

extern "C" gptq_status gptq_hptq_encode(const int16_t* levels, int64_t rows, int64_t cols,
                                        uint8_t* code_len, uint32_t* words,
                                        int64_t capacity_words, int64_t* row_bit,
                                        int64_t* total_bits, void* ws, size_t ws_bytes,
                                        void* stream) {
  if (rows < 0 || cols < 0 || capacity_words < 0 || !row_bit || !total_bits) return GPTQ_EINVAL;
  if (rows > 0 && cols > 0 && !levels) return GPTQ_EINVAL;
  if (capacity_words > 0 && !words) return GPTQ_EINVAL;
  if (cols > (int64_t)1 << 24 || rows > (int64_t)1 << 26) return GPTQ_EINVAL;
  const HFLayout L;
  if (!ws || ws_bytes < L.total) return GPTQ_EWORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  char* base = (char*)ws;
  unsigned* hist = (unsigned*)(base + L.hist);
  uint8_t* dlen = (uint8_t*)(base + L.len);
  uint64_t* dcode = (uint64_t*)(base + L.code);
  const int64_t n = rows * cols;
  GPTQ_LAUNCH(K_HF, st, hf_zero_kernel<<<64, 256, 0, st>>>(hist, HF_SYMS));
  if (n > 0)
    GPTQ_LAUNCH(K_HF, st,
                hf_hist_kernel<<<(unsigned)std::min<int64_t>(cdiv(n, 256), 8192), 256, 0, st>>>(
                    levels, n, hist));
  std::vector<unsigned> h(HF_SYMS);
  GPTQ_HIP(hipMemcpyAsync(h.data(), hist, sizeof(unsigned) * HF_SYMS, hipMemcpyDeviceToHost, st));
  GPTQ_HIP(hipStreamSynchronize(st));
  std::vector<uint8_t> len;
  if (!hf_lengths(h, len)) return GPTQ_EINVAL;  // a code longer than 63 bits
  std::vector<uint64_t> code, first;
  std::vector<int> count, index;
  std::vector<int16_t> sorted;
  hf_canonical(len, code, first, count, index, sorted);
  GPTQ_HIP(hipMemcpyAsync(dlen, len.data(), HF_SYMS, hipMemcpyHostToDevice, st));
  GPTQ_HIP(hipMemcpyAsync(dcode, code.data(), 8 * (size_t)HF_SYMS, hipMemcpyHostToDevice, st));
  const unsigned nb = (unsigned)cdiv(rows, 4);
  if (rows > 0)
    GPTQ_LAUNCH(K_HF, st, hf_rowbits_kernel<<<nb, 256, 0, st>>>(levels, rows, cols, dlen,
                                                                  row_bit));
  GPTQ_LAUNCH(K_HF, st, hf_scan_kernel<<<1, 1024, 0, st>>>(row_bit, rows));
  int64_t total = 0;
  GPTQ_HIP(hipMemcpyAsync(&total, row_bit + rows, sizeof(int64_t), hipMemcpyDeviceToHost, st));
  GPTQ_HIP(hipStreamSynchronize(st));  // the host vectors above are read by now too
  *total_bits = total;
  if (code_len) std::copy(len.begin(), len.end(), code_len);
  const int64_t need = cdiv(total, 32);
  if (need > capacity_words) return GPTQ_EINVAL;  // row_bit and total_bits are set
  if (need > 0) {
    GPTQ_LAUNCH(K_HF, st,
                hf_zero_kernel<<<(unsigned)std::min<int64_t>(cdiv(need, 256), 8192), 256, 0, st>>>(
                    words, need));
    GPTQ_LAUNCH(K_HF, st, hf_encode_kernel<<<nb, 256, 0, st>>>(levels, rows, cols, dlen, dcode,
                                                                 row_bit, words));
  }
  GPTQ_HIP(hipStreamSynchronize(st));
  return GPTQ_OK;
}

extern "C" gptq_status gptq_hptq_decode(const uint32_t* words, int64_t nwords,
                                        const int64_t* row_bit, int64_t rows, int64_t cols,
                                        const uint8_t* code_len, int16_t* levels, void* ws,
                                        size_t ws_bytes, void* stream) {
  if (rows < 0 || cols < 0 || nwords < 0 || !code_len || !row_bit) return GPTQ_EINVAL;
  if (rows > 0 && cols > 0 && (!words || !levels)) return GPTQ_EINVAL;
  if (cols > (int64_t)1 << 24 || rows > (int64_t)1 << 26) return GPTQ_EINVAL;
  const HFLayout L;
  if (!ws || ws_bytes < L.total) return GPTQ_EWORKSPACE;
  for (int s = 0; s < HF_SYMS; ++s)
    if (code_len[s] > HF_MAXLEN) return GPTQ_EINVAL;
  if (rows == 0 || cols == 0) return GPTQ_OK;
  hipStream_t st = (hipStream_t)stream;
  char* base = (char*)ws;
  std::vector<uint8_t> len(code_len, code_len + HF_SYMS);
  std::vector<uint64_t> code, first;
  std::vector<int> count, index;
  std::vector<int16_t> sorted;
  hf_canonical(len, code, first, count, index, sorted);
  if (sorted.empty()) return GPTQ_EINVAL;
  unsigned* bad = (unsigned*)(base + L.hist);
  uint64_t* dfirst = (uint64_t*)(base + L.first);
  int* dcount = (int*)(base + L.count);
  int* dindex = (int*)(base + L.index);
  int16_t* dsorted = (int16_t*)(base + L.sorted);
  GPTQ_HIP(hipMemcpyAsync(dfirst, first.data(), 8 * first.size(), hipMemcpyHostToDevice, st));
  GPTQ_HIP(hipMemcpyAsync(dcount, count.data(), 4 * count.size(), hipMemcpyHostToDevice, st));
  GPTQ_HIP(hipMemcpyAsync(dindex, index.data(), 4 * index.size(), hipMemcpyHostToDevice, st));
  GPTQ_HIP(hipMemcpyAsync(dsorted, sorted.data(), 2 * sorted.size(), hipMemcpyHostToDevice, st));
  GPTQ_LAUNCH(K_HF, st, hf_zero_kernel<<<1, 64, 0, st>>>(bad, 1));
  GPTQ_LAUNCH(K_HF, st,
              hf_decode_kernel<<<(unsigned)cdiv(rows, 256), 256, 0, st>>>(
                  words, nwords, row_bit, rows, cols, dfirst, dcount, dindex, dsorted, levels,
                  bad));
  unsigned hb = 0;
  GPTQ_HIP(hipMemcpyAsync(&hb, bad, sizeof(unsigned), hipMemcpyDeviceToHost, st));
  GPTQ_HIP(hipStreamSynchronize(st));  // the host tables above are read by now too
  return hb ? GPTQ_EINVAL : GPTQ_OK;
}
