// Reading a profiled cost table C_est(rows, len) from its JSON file (host).
//
// CoDec: Prefix-Shared Decoding Kernel for LLMs, section 工作负载平衡
// (workload balance): the partial-attention kernel is profiled over a grid of
// shapes on the target hardware and the planner interpolates that table.  The
// fitted gfx950 tables ship as JSON objects whose keys "rows_grid" and
// "len_grid" hold ascending integer grids and "table_ns" the row-major table
// (one array per rows point) in integer nanoseconds; other keys are notes and
// are skipped.  The parser below accepts standard JSON (RFC 8259) and keeps
// only those three arrays.
#include <cctype>
#include <cerrno>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "pst_internal.h"

namespace pst {
namespace {

class Json {
 public:
  explicit Json(const std::string& s) : s_(s) {}

  // Parses the top-level object; fills the three arrays it finds.
  bool parse_table(std::vector<int64_t>* rows, std::vector<int64_t>* lens, std::vector<std::vector<int64_t>>* table,
                   bool* have_rows, bool* have_lens, bool* have_table) {
    ws();
    if (!eat('{')) return fail("the file does not hold a JSON object");
    ws();
    if (eat('}')) return done();
    for (;;) {
      ws();
      std::string key;
      if (!string(&key)) return false;
      ws();
      if (!eat(':')) return fail("':' expected after a key");
      ws();
      if (key == "rows_grid") {
        if (!int_array(rows)) return false;
        *have_rows = true;
      } else if (key == "len_grid") {
        if (!int_array(lens)) return false;
        *have_lens = true;
      } else if (key == "table_ns") {
        if (!eat('[')) return fail("table_ns must be an array of arrays");
        table->clear();
        ws();
        if (!eat(']')) {
          for (;;) {
            ws();
            table->emplace_back();
            if (!int_array(&table->back())) return false;
            ws();
            if (eat(']')) break;
            if (!eat(',')) return fail("',' or ']' expected in table_ns");
          }
        }
        *have_table = true;
      } else if (!skip_value()) {
        return false;
      }
      ws();
      if (eat('}')) return done();
      if (!eat(',')) return fail("',' or '}' expected in the object");
    }
  }

  const std::string& error() const { return err_; }

 private:
  const std::string& s_;
  size_t i_ = 0;
  std::string err_;

  bool fail(const std::string& m) {
    if (err_.empty()) err_ = m + " (at byte " + std::to_string(i_) + ")";
    return false;
  }
  bool done() {
    ws();
    return i_ == s_.size() ? true : fail("trailing characters after the object");
  }
  void ws() {
    while (i_ < s_.size() && (s_[i_] == ' ' || s_[i_] == '\t' || s_[i_] == '\n' || s_[i_] == '\r')) ++i_;
  }
  bool eat(char c) {
    if (i_ < s_.size() && s_[i_] == c) {
      ++i_;
      return true;
    }
    return false;
  }
  bool literal(const char* w) {
    size_t k = 0;
    while (w[k]) {
      if (i_ + k >= s_.size() || s_[i_ + k] != w[k]) return fail("invalid literal");
      ++k;
    }
    i_ += k;
    return true;
  }
  bool string(std::string* out) {
    if (!eat('"')) return fail("a string was expected");
    for (;;) {
      if (i_ >= s_.size()) return fail("unterminated string");
      const char c = s_[i_++];
      if (c == '"') return true;
      if (static_cast<unsigned char>(c) < 0x20) return fail("control character in a string");
      if (c == '\\') {
        if (i_ >= s_.size()) return fail("unterminated escape");
        const char e = s_[i_++];
        if (e == 'u') {
          for (int k = 0; k < 4; ++k, ++i_)
            if (i_ >= s_.size() || !std::isxdigit(static_cast<unsigned char>(s_[i_]))) return fail("bad \\u escape");
          if (out) out->push_back('?');  // keys compared here are plain ASCII
        } else if (e == '"' || e == '\\' || e == '/' || e == 'b' || e == 'f' || e == 'n' || e == 'r' || e == 't') {
          if (out) out->push_back(e);
        } else {
          return fail("bad escape");
        }
      } else if (out) {
        out->push_back(c);
      }
    }
  }
  // A JSON number; *is_int tells whether it is an integer in int64 range.
  bool number(double* val, int64_t* ival, bool* is_int) {
    const size_t b = i_;
    eat('-');
    if (i_ >= s_.size() || !std::isdigit(static_cast<unsigned char>(s_[i_]))) return fail("a number was expected");
    if (s_[i_] == '0') {
      ++i_;
    } else {
      while (i_ < s_.size() && std::isdigit(static_cast<unsigned char>(s_[i_]))) ++i_;
    }
    bool frac = false;
    if (eat('.')) {
      frac = true;
      if (i_ >= s_.size() || !std::isdigit(static_cast<unsigned char>(s_[i_]))) return fail("digits expected after '.'");
      while (i_ < s_.size() && std::isdigit(static_cast<unsigned char>(s_[i_]))) ++i_;
    }
    if (i_ < s_.size() && (s_[i_] == 'e' || s_[i_] == 'E')) {
      frac = true;
      ++i_;
      if (!eat('+')) eat('-');
      if (i_ >= s_.size() || !std::isdigit(static_cast<unsigned char>(s_[i_]))) return fail("bad exponent");
      while (i_ < s_.size() && std::isdigit(static_cast<unsigned char>(s_[i_]))) ++i_;
    }
    const std::string tok = s_.substr(b, i_ - b);
    *val = std::strtod(tok.c_str(), nullptr);
    *is_int = false;
    if (!frac) {
      errno = 0;
      const long long v = std::strtoll(tok.c_str(), nullptr, 10);
      if (errno == 0) {
        *ival = v;
        *is_int = true;
      }
    }
    return true;
  }
  bool int_array(std::vector<int64_t>* out) {
    if (!eat('[')) return fail("an array of integers was expected");
    out->clear();
    ws();
    if (eat(']')) return true;
    for (;;) {
      ws();
      double d = 0;
      int64_t v = 0;
      bool is_int = false;
      if (!number(&d, &v, &is_int)) return false;
      if (!is_int) return fail("a grid or table entry is not an integer");
      out->push_back(v);
      ws();
      if (eat(']')) return true;
      if (!eat(',')) return fail("',' or ']' expected in an array");
    }
  }
  bool skip_value(int depth = 0) {
    if (depth > 64) return fail("nesting too deep");
    ws();
    if (i_ >= s_.size()) return fail("a value was expected");
    const char c = s_[i_];
    if (c == '"') return string(nullptr);
    if (c == 't') return literal("true");
    if (c == 'f') return literal("false");
    if (c == 'n') return literal("null");
    if (c == '[' || c == '{') {
      const char close = c == '[' ? ']' : '}';
      ++i_;
      ws();
      if (eat(close)) return true;
      for (;;) {
        ws();
        if (c == '{') {
          if (!string(nullptr)) return false;
          ws();
          if (!eat(':')) return fail("':' expected after a key");
        }
        if (!skip_value(depth + 1)) return false;
        ws();
        if (eat(close)) return true;
        if (!eat(',')) return fail("',' expected");
      }
    }
    double d;
    int64_t v;
    bool is_int;
    return number(&d, &v, &is_int);
  }
};

}  // namespace

pst_status load_cost_json(const char* path, std::vector<int32_t>* rows_grid, std::vector<int32_t>* len_grid,
                          std::vector<int64_t>* table) {
  std::FILE* f = std::fopen(path, "rb");
  if (!f) {
    set_error(std::string("cannot open cost table ") + path);
    return PST_E_INVALID_ARG;
  }
  std::string text;
  char buf[65536];
  size_t n;
  while ((n = std::fread(buf, 1, sizeof buf, f)) > 0) text.append(buf, n);
  const bool read_error = std::ferror(f) != 0;
  std::fclose(f);
  if (read_error) {
    set_error(std::string("cannot read cost table ") + path);
    return PST_E_INVALID_ARG;
  }
  std::vector<int64_t> rows, lens;
  std::vector<std::vector<int64_t>> tab;
  bool hr = false, hl = false, ht = false;
  Json j(text);
  if (!j.parse_table(&rows, &lens, &tab, &hr, &hl, &ht)) {
    set_error(std::string("cost table ") + path + ": " + j.error());
    return PST_E_INVALID_ARG;
  }
  if (!hr || !hl || !ht) {
    set_error(std::string("cost table ") + path + ": rows_grid, len_grid and table_ns are required");
    return PST_E_INVALID_ARG;
  }
  if (tab.size() != rows.size()) {
    set_error(std::string("cost table ") + path + ": table_ns needs one array per rows_grid point");
    return PST_E_INVALID_ARG;
  }
  for (const int64_t v : rows)
    if (v < 1 || v > INT32_MAX) {
      set_error(std::string("cost table ") + path + ": rows_grid entries must lie in [1, 2^31 - 1]");
      return PST_E_INVALID_ARG;
    }
  for (const int64_t v : lens)
    if (v < 1 || v > INT32_MAX) {
      set_error(std::string("cost table ") + path + ": len_grid entries must lie in [1, 2^31 - 1]");
      return PST_E_INVALID_ARG;
    }
  rows_grid->assign(rows.begin(), rows.end());
  len_grid->assign(lens.begin(), lens.end());
  table->clear();
  for (const auto& r : tab) {
    if (r.size() != lens.size()) {
      set_error(std::string("cost table ") + path + ": every table_ns row needs one entry per len_grid point");
      return PST_E_INVALID_ARG;
    }
    table->insert(table->end(), r.begin(), r.end());
  }
  return PST_OK;
}

}  // namespace pst
