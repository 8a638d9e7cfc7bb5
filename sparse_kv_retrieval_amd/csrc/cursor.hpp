// Wave-uniform walk over the 64-entry mask words of the score pass.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace lsa {

// Sequence table lookups go through the constant address space: the table is
// read-only in these kernels, so with a wave-uniform index each lookup is a
// scalar load. It waits only on the scalar/LDS counter, never on the vector
// loads that stream the keys.
typedef const __attribute__((address_space(4))) int64_t* seq_ptr;

struct SeqTab {
  seq_ptr koff;
  seq_ptr mwo;
  __device__ __forceinline__ SeqTab(const int64_t* k, const int64_t* m) : koff((seq_ptr)k), mwo((seq_ptr)m) {}
};

// Largest b in [0, n) with off[b] <= x, given off[0] <= x < off[n] and off
// non-decreasing (skips empty sequences).
__device__ __forceinline__ int seq_upper(seq_ptr off, int n, int64_t x) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= x) lo = mid; else hi = mid;
  }
  return lo;
}

// Wave-uniform cursor over the mask words of one wave: (layer, sequence, word).
// It advances one word at a time, so there is no division or search in the
// steady state. A search runs only when the cursor is placed.
struct WordCursor {
  int l, b;
  int64_t word;     // word index in the mask layout
  int64_t seq_hi;   // first word after sequence b
  int32_t e0;       // entry index (within sequence b) of the word's first bit
  int32_t nb;       // sequence b's entry count (< 2^31, checked on the host)
  int64_t row0;     // sequence b's first key row
  // layer l's buffers, read from the arguments only when the layer changes
  // (past the last layer: the last layer's, never dereferenced)
  const char* keys;
  const float* scale;
  uint64_t* mask;
  float* score;

  __device__ __forceinline__ void load_layer(const ScoreArgs& a) {
    const int ll = l < a.L ? l : a.L - 1;
    keys = (const char*)a.keys[ll];
    scale = a.scale[ll];
    mask = a.mask[ll];
    score = a.score[ll];
  }
  __device__ __forceinline__ void load_seq(const SeqTab& t) {
    const int64_t lo = uni(t.mwo[b]);
    seq_hi = uni(t.mwo[b + 1]);
    row0 = uni(t.koff[b]);
    nb = uni((int32_t)(uni(t.koff[b + 1]) - row0));
    e0 = uni((int32_t)((word - lo) * 64));
  }
  __device__ __forceinline__ void place(const ScoreArgs& a, const SeqTab& t, int64_t gw) {
    l = uni((int32_t)(gw / a.words_per_layer));
    word = uni(a.word_base + (gw - (int64_t)l * a.words_per_layer));
    b = uni(seq_upper(t.mwo, a.B, word));
    load_seq(t);
    load_layer(a);
  }
  __device__ __forceinline__ void next(const ScoreArgs& a, const SeqTab& t) {
    ++word;
    e0 += 64;
    if (word == seq_hi) {
      if (word == a.word_base + a.words_per_layer) {
        ++l;
        word = a.word_base;
        b = 0;
        load_layer(a);
      } else {
        ++b;
      }
      while (uni(t.mwo[b + 1]) == uni(t.mwo[b])) ++b;  // skip empty sequences
      load_seq(t);
    }
  }
  // Move to global word gw (layer-major word index) at or after the current
  // one. Inside the current sequence this is O(1); otherwise it places anew.
  __device__ __forceinline__ void jump(const ScoreArgs& a, const SeqTab& t, int64_t gw) {
    const int64_t lbase = (int64_t)l * a.words_per_layer - a.word_base;
    const int64_t cur = lbase + word, end = lbase + seq_hi;
    if (gw >= cur && gw < end) {
      const int64_t d = gw - cur;
      word += d;
      e0 += (int32_t)(64 * d);
    } else {
      place(a, t, gw);
    }
  }
  __device__ __forceinline__ void advance(const ScoreArgs& a, const SeqTab& t, int g) {
    for (int i = 0; i < g; ++i) next(a, t);
  }
};

}  // namespace lsa
