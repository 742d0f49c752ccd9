// SHA-256 (FIPS 180-4), written from the standard's definition: 512-bit
// blocks, the 64-word message schedule, 64 rounds of the compression
// function, big-endian length padding.  The round constants (fractional
// parts of the cube roots of the first 64 primes) and the initial hash value
// (fractional parts of the square roots of the first 8 primes) are computed
// here with exact integer roots rather than written out.
#pragma once

#include <cstddef>
#include <cstdint>
#include <cstring>

namespace pkv {

class Sha256 {
 public:
  Sha256() { reset(); }

  void reset() {
    const Tables& t = tables();
    std::memcpy(h_, t.h0, sizeof h_);
    bytes_ = 0;
    fill_ = 0;
  }

  void update(const void* data, size_t n) {
    const uint8_t* p = static_cast<const uint8_t*>(data);
    bytes_ += n;
    while (n > 0) {
      const size_t take = (64 - fill_) < n ? (64 - fill_) : n;
      std::memcpy(buf_ + fill_, p, take);
      fill_ += take;
      p += take;
      n -= take;
      if (fill_ == 64) {
        compress(buf_);
        fill_ = 0;
      }
    }
  }

  void finish(uint8_t out[32]) {
    const uint64_t bits = bytes_ * 8;
    buf_[fill_++] = 0x80;
    if (fill_ > 56) {   // no room for the length: pad out this block
      std::memset(buf_ + fill_, 0, 64 - fill_);
      compress(buf_);
      fill_ = 0;
    }
    std::memset(buf_ + fill_, 0, 56 - fill_);
    for (int i = 0; i < 8; ++i) buf_[56 + i] = static_cast<uint8_t>(bits >> (56 - 8 * i));
    compress(buf_);
    fill_ = 0;
    for (int i = 0; i < 8; ++i)
      for (int j = 0; j < 4; ++j) out[4 * i + j] = static_cast<uint8_t>(h_[i] >> (24 - 8 * j));
  }

 private:
  struct Tables {
    uint32_t k[64];
    uint32_t h0[8];
  };

  static unsigned __int128 iroot(unsigned __int128 x, int degree) {
    // largest r with r^degree <= x; here x < 2^105 and degree >= 2, so r < 2^40
    // and r^3 < 2^120 stays inside 128 bits
    uint64_t lo = 0, hi = uint64_t(1) << 40;
    while (hi - lo > 1) {
      const uint64_t mid = lo + (hi - lo) / 2;
      unsigned __int128 p = mid;
      for (int d = 1; d < degree; ++d) p *= mid;
      if (p <= x) lo = mid; else hi = mid;
    }
    return lo;
  }

  static const Tables& tables() {
    static const Tables t = [] {
      Tables r{};
      int primes[64];
      int n = 0;
      for (int c = 2; n < 64; ++c) {
        bool prime = true;
        for (int d = 2; d * d <= c; ++d)
          if (c % d == 0) { prime = false; break; }
        if (prime) primes[n++] = c;
      }
      for (int i = 0; i < 64; ++i)  // floor(cbrt(p) * 2^32) = icbrt(p * 2^96); keep the low 32 bits
        r.k[i] = static_cast<uint32_t>(iroot(static_cast<unsigned __int128>(primes[i]) << 96, 3));
      for (int i = 0; i < 8; ++i)   // floor(sqrt(p) * 2^32) = isqrt(p * 2^64)
        r.h0[i] = static_cast<uint32_t>(iroot(static_cast<unsigned __int128>(primes[i]) << 64, 2));
      return r;
    }();
    return t;
  }

  static uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

  void compress(const uint8_t* blk) {
    const Tables& t = tables();
    uint32_t w[64];
    for (int i = 0; i < 16; ++i)
      w[i] = (uint32_t(blk[4 * i]) << 24) | (uint32_t(blk[4 * i + 1]) << 16) | (uint32_t(blk[4 * i + 2]) << 8) |
             uint32_t(blk[4 * i + 3]);
    for (int i = 16; i < 64; ++i) {
      const uint32_t s0 = rotr(w[i - 15], 7) ^ rotr(w[i - 15], 18) ^ (w[i - 15] >> 3);
      const uint32_t s1 = rotr(w[i - 2], 17) ^ rotr(w[i - 2], 19) ^ (w[i - 2] >> 10);
      w[i] = w[i - 16] + s0 + w[i - 7] + s1;
    }
    uint32_t a = h_[0], b = h_[1], c = h_[2], d = h_[3], e = h_[4], f = h_[5], g = h_[6], h = h_[7];
    for (int i = 0; i < 64; ++i) {
      const uint32_t big1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
      const uint32_t choose = (e & f) ^ (~e & g);
      const uint32_t t1 = h + big1 + choose + t.k[i] + w[i];
      const uint32_t big0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
      const uint32_t majority = (a & b) ^ (a & c) ^ (b & c);
      const uint32_t t2 = big0 + majority;
      h = g;
      g = f;
      f = e;
      e = d + t1;
      d = c;
      c = b;
      b = a;
      a = t1 + t2;
    }
    h_[0] += a;
    h_[1] += b;
    h_[2] += c;
    h_[3] += d;
    h_[4] += e;
    h_[5] += f;
    h_[6] += g;
    h_[7] += h;
  }

  uint32_t h_[8];
  uint64_t bytes_;
  uint8_t buf_[64];
  size_t fill_;
};

}  // namespace pkv
