// Error text shared by the library's source files: the message that
// gpt2_last_error(NULL) returns for calls that have no model handle.
#pragma once
#include <string>

void set_last_error(const std::string &msg);
