// SHA-256 (FIPS 180-4) for the prefix cache's block digests.
//
// The 64 round constants are the first 32 fractional bits of the cube roots
// of the first 64 primes and the initial state the first 32 fractional bits
// of the square roots of the first 8 primes (FIPS 180-4, 4.2.2 and 5.3.3).
// They are computed once from that definition: a floating-point estimate of
// floor(root(p) * 2^32), corrected with exact 128-bit integer arithmetic so
// that m^k <= p * 2^(32k) < (m+1)^k holds, then reduced mod 2^32.
#pragma once

#include <array>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstring>

#if !defined(__BYTE_ORDER__) || __BYTE_ORDER__ != __ORDER_LITTLE_ENDIAN__
#error "block digests hash int32 token ids in host byte order, which must be little-endian"
#endif

namespace pkv {

using Digest = std::array<uint8_t, 32>;

namespace sha256_detail {

using u128 = unsigned __int128;

// floor(p^(1/k) * 2^32) mod 2^32 for k = 2 or 3, exactly.
inline uint32_t root_fraction_bits(uint32_t p, int k) {
  const u128 target = static_cast<u128>(p) << (32 * k);
  const long double est = (k == 2 ? std::sqrt(static_cast<long double>(p)) : std::cbrt(static_cast<long double>(p))) *
                          4294967296.0L;
  u128 m = static_cast<u128>(est);
  auto pw = [k](u128 x) { return k == 2 ? x * x : x * x * x; };
  while (pw(m) > target) --m;
  while (pw(m + 1) <= target) ++m;
  return static_cast<uint32_t>(m & 0xFFFFFFFFu);
}

struct Constants {
  uint32_t k[64];
  uint32_t h0[8];
  Constants() {
    int found = 0;
    for (uint32_t n = 2; found < 64; ++n) {
      bool prime = true;
      for (uint32_t d = 2; d * d <= n; ++d)
        if (n % d == 0) {
          prime = false;
          break;
        }
      if (!prime) continue;
      if (found < 8) h0[found] = root_fraction_bits(n, 2);
      k[found++] = root_fraction_bits(n, 3);
    }
  }
};

inline const Constants& constants() {
  static const Constants c;
  return c;
}

inline uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

inline void compress(uint32_t st[8], const uint8_t* blk, const uint32_t* K) {
  uint32_t w[64];
  for (int t = 0; t < 16; ++t)
    w[t] = (uint32_t(blk[4 * t]) << 24) | (uint32_t(blk[4 * t + 1]) << 16) | (uint32_t(blk[4 * t + 2]) << 8) |
           uint32_t(blk[4 * t + 3]);
  for (int t = 16; t < 64; ++t) {
    const uint32_t s0 = rotr(w[t - 15], 7) ^ rotr(w[t - 15], 18) ^ (w[t - 15] >> 3);
    const uint32_t s1 = rotr(w[t - 2], 17) ^ rotr(w[t - 2], 19) ^ (w[t - 2] >> 10);
    w[t] = s1 + w[t - 7] + s0 + w[t - 16];
  }
  uint32_t a = st[0], b = st[1], c = st[2], d = st[3], e = st[4], f = st[5], g = st[6], h = st[7];
  for (int t = 0; t < 64; ++t) {
    const uint32_t big1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
    const uint32_t ch = (e & f) ^ (~e & g);
    const uint32_t t1 = h + big1 + ch + K[t] + w[t];
    const uint32_t big0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
    const uint32_t maj = (a & b) ^ (a & c) ^ (b & c);
    const uint32_t t2 = big0 + maj;
    h = g;
    g = f;
    f = e;
    e = d + t1;
    d = c;
    c = b;
    b = a;
    a = t1 + t2;
  }
  st[0] += a;
  st[1] += b;
  st[2] += c;
  st[3] += d;
  st[4] += e;
  st[5] += f;
  st[6] += g;
  st[7] += h;
}

}  // namespace sha256_detail

// Streaming SHA-256: update() any number of times, then finish().
class Sha256 {
 public:
  Sha256() {
    const auto& c = sha256_detail::constants();
    std::memcpy(st_, c.h0, sizeof(st_));
  }
  void update(const void* data, size_t n) {
    const auto* p = static_cast<const uint8_t*>(data);
    const uint32_t* K = sha256_detail::constants().k;
    total_ += n;
    while (n > 0) {
      const size_t take = n < 64 - fill_ ? n : 64 - fill_;
      std::memcpy(buf_ + fill_, p, take);
      fill_ += take;
      p += take;
      n -= take;
      if (fill_ == 64) {
        sha256_detail::compress(st_, buf_, K);
        fill_ = 0;
      }
    }
  }
  Digest finish() {
    // Padding: one 1 bit, zeros up to 56 mod 64 bytes, then the bit length
    // as a 64-bit big-endian integer.
    const uint64_t bits = static_cast<uint64_t>(total_) * 8;
    uint8_t pad[72] = {0x80};
    const size_t zeros = (fill_ < 56 ? 56 - fill_ : 120 - fill_) - 1;
    for (int i = 0; i < 8; ++i) pad[1 + zeros + i] = static_cast<uint8_t>(bits >> (56 - 8 * i));
    update(pad, 1 + zeros + 8);
    Digest d;
    for (int i = 0; i < 8; ++i)
      for (int j = 0; j < 4; ++j) d[4 * i + j] = static_cast<uint8_t>(st_[i] >> (24 - 8 * j));
    return d;
  }

 private:
  uint32_t st_[8];
  uint8_t buf_[64];
  size_t fill_ = 0;
  size_t total_ = 0;
};

// Chain digest of one full block: SHA-256(parent || salt (8 bytes,
// little-endian) || token ids (int32, little-endian)).
inline Digest block_digest(const Digest& parent, uint64_t salt, const int32_t* tokens, int32_t n) {
  Sha256 h;
  h.update(parent.data(), parent.size());
  uint8_t s[8];
  for (int i = 0; i < 8; ++i) s[i] = static_cast<uint8_t>(salt >> (8 * i));
  h.update(s, 8);
  h.update(tokens, static_cast<size_t>(n) * 4);  // int32 in host order = little-endian
  return h.finish();
}

struct DigestHash {
  size_t operator()(const Digest& d) const {
    size_t v;
    std::memcpy(&v, d.data(), sizeof(v));
    return v;
  }
};

}  // namespace pkv
